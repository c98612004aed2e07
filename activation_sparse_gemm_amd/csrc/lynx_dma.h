// Device helpers shared by the kernels that stage operands with LDS-DMA
// (buffer_load ... lds): buffer resources, the DMA instructions and explicit
// vmcnt waits.  Internal; not installed.
#pragma once

#include "lynx_internal.h"

namespace lynx {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit format

// Buffer resource over `bytes` bytes at `base` (accesses past it read zero and
// write nothing; the range check covers the VGPR offset only).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{int(uint32_t(p)), int(uint32_t(p >> 32) & 0xFFFFu), int(bytes), kRsrcWord3};
}

// One wave-wide global -> LDS copy: lane l's 16 (or 4) bytes at
// rsrc + voff + soff land at LDS byte lds + 16 l (or 4 l).  The buffer range
// check covers voff only, so voff carries the row and soff the k offset (a
// row inside the buffer stays inside it at every k).  Offsets are unsigned
// 32-bit byte offsets; the shape limits keep every padded row below 2^32.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) (n < 64), leaving lgkmcnt / expcnt alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(n) lgkmcnt(0): own LDS reads done, vector loads down to n
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// s_waitcnt lgkmcnt(0) alone
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(0x3F | (0x7 << 4) | (0x3 << 14));
}

// LDS byte address of a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

}  // namespace lynx
