// Device helpers shared by the tiled GEMM kernels (k_gemm.hip, K2;
// k_gemm_dense.hip, K3): tile geometry, LDS swizzles, the XCD-aware tile
// order and the direct-store epilogue.  Internal; not installed.
#pragma once

#include "lynx_dma.h"

namespace lynx {

constexpr int BM = 256, NT = 256, GROUP_M = 8;

// 16-byte chunk swizzles within 64-byte and 128-byte rows
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz128(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = ntiles >> 3, rem = ntiles & 7;
    const int v = xcd * per + min(xcd, rem) + slot;
    const int group_size = GROUP_M * tiles_n;
    const int group = v / group_size;
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in = v - group * group_size;
    tm = first_m + in % gm;
    tn = in / gm;
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The lane id, computed afresh where it is called: per-lane constants needed
// only at tile boundaries are then recomputed there instead of being kept
// live (and spilled) across the main loop.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

template <typename T>
__device__ __forceinline__ T lds_read(const char* smem, int off) {
    return *reinterpret_cast<const T*>(smem + off);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
           (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Stores one wave's 128 x 32 NB output block straight from the accumulators,
// for tiles whose columns all lie inside N (N % 8 == 0).  A lane holds one
// column of each 32 x 32 tile, rows 8 (e / 4) + 4 h + e % 4.  Rows e and e + 1
// (e even) are converted together; the pair is swapped with the neighbouring
// column's lane (DPP quad permute) and each lane keeps one row of both
// columns: even columns row e, odd columns row e + 1.  Each store writes two
// adjacent outputs, and a half-wave's 16 lanes cover 64 contiguous bytes of a
// row.  The whole byte offset, row part included, goes in the VGPR offset,
// which the buffer range check covers (the SGPR offset is not checked): rows
// past M lie past the end of the buffer resource and are dropped.  The shape
// limits keep (M + 256) N < 2^31, so the offsets of those rows cannot wrap.
// row0, col0: the block's first output row and column.
template <int NB>
__device__ __forceinline__ void store_block_direct(const f32x16 (&acc)[4][NB],
                                                   __amdgpu_buffer_rsrc_t rsY, int N, int row0,
                                                   int col0) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const int el = fresh_lane();
    const int er = el & 31, eh = el >> 5;
    // v_perm_b32 selectors over {partner pair : own pair}: even columns take
    // the low halves (row e of own and partner column), odd the high halves
    const uint32_t psel = (er & 1) ? 0x03020706u : 0x05040100u;
    const uint32_t vbase =
        (uint32_t(row0 + 4 * eh + (er & 1)) * uint32_t(N) + uint32_t(col0 + (er & ~1))) * 2u;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const uint32_t own = __builtin_bit_cast(
                    uint32_t,
                    __builtin_convertvector(f32x2_t{acc[a][b][e], acc[a][b][e + 1]}, bf16x2_t));
                const uint32_t partner =
                    uint32_t(__builtin_amdgcn_update_dpp(0, int(own), 0xB1, 0xF, 0xF, false));
                const uint32_t w = __builtin_amdgcn_perm(partner, own, psel);
                const uint32_t roff =
                    (uint32_t(32 * a + 8 * (e / 4) + (e % 4)) * uint32_t(N) + uint32_t(32 * b)) * 2u;
                __builtin_amdgcn_raw_buffer_store_b32(w, rsY, vbase + roff, 0, 0);
            }
}


}  // namespace lynx
