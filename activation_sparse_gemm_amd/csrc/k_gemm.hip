// Tiled GEMM kernels for gfx950: K2 (2:4 sparse MFMA + LoRA epilogue) and K3
// (dense MFMA baseline), sharing one tile pipeline.
//
// Layer (RT-Lynx page, 코드 예제, second formula; 방법론 "핵심 메커니즘" and
// "CUDA 커널 최적화": the 2:4 activation goes to the sparse unit, the LoRA
// output is generated and accumulated on chip inside the sparse GEMM):
//   Y = s * (X~ W^T) + T LA^T = s * (X~ W^T + (T / s) LA^T).
// The second form lets the LoRA up-projection accumulate into the same fp32
// accumulators as the sparse product, with one multiply by s per output in the
// epilogue; T / s is rounded to bf16 once when staged (its share of Y is a few
// per mille, so that rounding is far below the output's own bf16 rounding).
//
// Tiling: one 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave
// 128 x 128 = 8 x 8 accumulator tiles of 16 x 16 (256 fp32 per lane, in AGPRs).
// Operands move global -> LDS by buffer_load ... lds (no VGPR staging) into a
// ring of LDS stages of 64 dense channels:
//   sparse: A = packed values 256 x 64 B, meta 256 x 8 B, B = W 256 x 128 B
//           (50 KB, 1024 matrix-core cycles per wave); ring of 3 (150 KB),
//           loads issued 2 stages ahead.  The packed operand is stored in
//           16-row x 64-channel tiles, so a stage's A side is 16 contiguous
//           1 KB value tiles and 16 contiguous 128 B meta tiles;
//   dense:  32 channels per stage: A = X 256 x 64 B, B = W 256 x 64 B
//           (32 KB, 1024 cycles); ring of 4 (128 KB), loads issued 3 ahead.
// The sparse A side is read as whole 128-byte lines, which keeps the L1 -> L2
// request rate (about one line per clock per CU) below the matrix-core rate.
// The loads of a stage are waited for with an explicit vmcnt that leaves the
// later stages' loads in flight, then one s_barrier per stage.  Rows past M or
// N lie past the end of their buffer resource and are never read (their LDS
// slots keep stale values, which only reach outputs that are not stored).
// LDS rows keep their 16-byte chunks XOR-swizzled by row so the fragment reads
// of 8 (and 16) consecutive lanes hit distinct banks.
//
// Register layouts (pinned by the probe tests), lane l, r = l % 16, q = l / 16:
//   v_smfmac_f32_16x16x64_bf16: A = row r, dense channels [16q, 16q+16) as 8
//     kept values + 16-bit index word; B = column r, channel chunks q and 4+q
//     (8 channels each) of the 64-channel step.
//   v_mfma_f32_16x16x32_bf16: A = row r, B = column r, channels [8q, 8q+8).
//   16 x 16 accumulator: column r, rows 4q .. 4q+3.
//
// Tile order: workgroups are handed to the 8 XCDs round-robin, so ids are
// remapped to give each XCD a contiguous range of tiles, and tiles are
// rasterized in groups of 8 tile-rows so the ~32 workgroups resident on one
// XCD share A rows and W rows in that XCD's L2.
#include "lynx_internal.h"

namespace lynx {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, NT = 256, GROUP_M = 8;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit format

template <bool SPARSE>
struct Cfg {
    static constexpr int BK = SPARSE ? 64 : 32;          // dense channels per stage
    static constexpr int A_ROW = 64;                     // LDS bytes per A row per stage
    static constexpr int B_ROW = SPARSE ? 128 : 64;      // LDS bytes per B row per stage
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int META_BYTES = SPARSE ? BM * 8 : 0;
    static constexpr int B_BYTES = BN * B_ROW;
    static constexpr int STAGE = A_BYTES + META_BYTES + B_BYTES;
    static constexpr int NSTAGE = SPARSE ? 3 : 4;
    static constexpr int A_DMA = A_BYTES / 1024 / 4;     // 1 KB DMA instructions per wave
    static constexpr int B_DMA = B_BYTES / 1024 / 4;
    static constexpr int M_DMA = META_BYTES / 256 / 4;   // 256 B (dword) DMA instructions
    static constexpr int DMA_PER_STAGE = A_DMA + B_DMA + M_DMA;
    static constexpr int EPI_OFF = 64 * 1024;            // epilogue scratch, 4 KB per wave
    static constexpr int SCALE_OFF = NSTAGE * STAGE;     // s of the tile's 256 rows (sparse)
    static constexpr int LDS = NSTAGE * STAGE + (SPARSE ? BM * 4 : 0);
    static_assert(LDS >= EPI_OFF + 4 * 4096, "epilogue scratch must fit");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(NSTAGE >= 3 && NSTAGE <= 4, "ring depth handled by the waits below");
    static_assert(NSTAGE * STAGE >= 64 * 1024 + 4 * 4096, "LoRA tiles and epilogue scratch");
    static_assert((NSTAGE - 1) * DMA_PER_STAGE < 64, "vmcnt range");
};

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

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{int(uint32_t(p)), int(uint32_t(p >> 32) & 0xFFFFu), int(bytes), kRsrcWord3};
}

// One wave-wide global -> LDS copy: lane l's 16 (or 4) bytes at
// rsrc + voff + soff land at LDS byte lds + 16 l (or 4 l).  The buffer range
// check covers voff only, so voff carries the row and soff the k offset.
__device__ __forceinline__ void dma16(uint32_t lds, int voff, i32x4 rsrc, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, int voff, i32x4 rsrc, int soff) {
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

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

template <bool SPARSE>
__global__ __launch_bounds__(NT, 1) void gemm_tiled(
    const uint16_t* __restrict__ Aptr,   // SPARSE: values [M][K/2]; dense: X [M][K]
    const uint8_t* __restrict__ meta,    // SPARSE only: [M][K/8]
    const float* __restrict__ scale,     // SPARSE only: [M]
    const uint16_t* __restrict__ T,      // SPARSE only: [M][R] or null
    const uint16_t* __restrict__ W,      // [N][K]
    const uint16_t* __restrict__ LA,     // SPARSE only: [N][R] or null
    uint16_t* __restrict__ Y, int M, int N, int K, int R) {
    using C = Cfg<SPARSE>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- DMA addressing --------------------------------------------------
    // sparse A: instruction j of wave w moves the 1 KB value tile of row block
    //   (m0/16 + w + 4j) into LDS rows 16 (w + 4j) .. +16 (64 B each);
    // sparse meta (dword DMA, 256 B): the two 128 B tiles of row blocks
    //   2 (w + 4j), 2 (w + 4j) + 1 into LDS rows 32 (w + 4j) .. +32 (8 B each);
    // sparse W (128-byte LDS rows): instruction j moves rows 8 (w + 4j) + l/8;
    // dense X and W (64-byte LDS rows): instruction j moves rows 16 (w + 4j) + l/4.
    // Lane l lands at LDS byte 16 l (4 l) of the instruction's 1 KB (256 B);
    // its source is the chunk the row's swizzle puts there.
    const uint32_t lds0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
    const int steps = K / 64;
    const int Mp = (M + 15) & ~15;
    const i32x4 rsA = SPARSE ? make_rsrc(Aptr, uint32_t(Mp) * uint32_t(K))
                             : make_rsrc(Aptr, uint32_t(M) * uint32_t(2 * K));
    const i32x4 rsB = make_rsrc(W, uint32_t(N) * uint32_t(2 * K));
    i32x4 rsM = {0, 0, 0, 0};
    if constexpr (SPARSE) rsM = make_rsrc(meta, uint32_t(Mp) * uint32_t(K / 8));

    int voffA[C::A_DMA], voffB[C::B_DMA], voffM[C::M_DMA > 0 ? C::M_DMA : 1];
#pragma unroll
    for (int j = 0; j < C::A_DMA; ++j) {
        if constexpr (SPARSE) {
            const int blk = wave + 4 * j, row = lane >> 2, ph = lane & 3;
            voffA[j] = (m0 / 16 + blk) * steps * 1024 + row * 64 + 16 * (ph ^ swz64(row));
        } else {
            const int row = 16 * (wave + 4 * j) + (lane >> 2), ph = lane & 3;
            voffA[j] = (m0 + row) * 2 * K + 16 * (ph ^ swz64(row));
        }
    }
#pragma unroll
    for (int j = 0; j < C::B_DMA; ++j) {
        if constexpr (SPARSE) {
            const int row = 8 * (wave + 4 * j) + (lane >> 3), ph = lane & 7;
            voffB[j] = (n0 + row) * 2 * K + 16 * (ph ^ swz128(row));
        } else {
            const int row = 16 * (wave + 4 * j) + (lane >> 2), ph = lane & 3;
            voffB[j] = (n0 + row) * 2 * K + 16 * (ph ^ swz64(row));
        }
    }
    if constexpr (SPARSE) {
#pragma unroll
        for (int j = 0; j < C::M_DMA; ++j) {
            const int blk = 2 * (wave + 4 * j) + (lane >> 5);
            voffM[j] = (m0 / 16 + blk) * steps * 128 + 4 * (lane & 31);
        }
    }

    // loads of k-stage t into ring slot t % NSTAGE (k offsets in bytes)
    auto issue_stage = [&](int t) {
        const uint32_t base = lds0 + uint32_t((t % C::NSTAGE) * C::STAGE);
        const int kA = SPARSE ? t * 1024 : t * 64;
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j) dma16(base + 1024 * (wave + 4 * j), voffA[j], rsA, kA);
        if constexpr (SPARSE) {
#pragma unroll
            for (int j = 0; j < C::M_DMA; ++j)
                dma4(base + C::A_BYTES + 256 * (wave + 4 * j), voffM[j], rsM, t * 128);
        }
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j)
            dma16(base + C::A_BYTES + C::META_BYTES + 1024 * (wave + 4 * j), voffB[j], rsB,
                  t * C::B_ROW);
    };

    // ---- per-lane fragment offsets (swizzle depends on row % 16 = r only) --
    const int s64 = swz64(r), s128 = swz128(r);
    (void)s64;
    const int rowA = wm * 128 + r, rowB = wn * 128 + r;

    f32x4 acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / C::BK;
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (SPARSE) {
        // s of the tile's 256 rows into LDS (rows past M repeat the last row)
        reinterpret_cast<float*>(smem + C::SCALE_OFF)[tid] = scale[min(m0 + tid, M - 1)];
    }

    // prologue: NSTAGE - 1 stages in flight
#pragma unroll
    for (int t = 0; t < C::NSTAGE - 1; ++t)
        if (t < nk) issue_stage(t);
    if (nk >= C::NSTAGE - 1) {
        wait_vmcnt<(C::NSTAGE - 2) * C::DMA_PER_STAGE>();
    } else {
        __builtin_amdgcn_s_waitcnt(0);
    }
    block_barrier();

    for (int t = 0; t < nk; ++t) {
        if (t + C::NSTAGE - 1 < nk) issue_stage(t + C::NSTAGE - 1);
        const char* cur = smem + (t % C::NSTAGE) * C::STAGE;
        if constexpr (SPARSE) {
            const char* As = cur;
            const char* Ms = cur + C::A_BYTES;
            const char* Bs = cur + C::A_BYTES + C::META_BYTES;
            bf16x16 bfr[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int base = (rowB + 16 * b) * 128;
                const bf16x8 lo = lds_read<bf16x8>(Bs, base + 16 * (q ^ s128));
                const bf16x8 hi = lds_read<bf16x8>(Bs, base + 16 * ((4 + q) ^ s128));
                bfr[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                                 12, 13, 14, 15);
            }
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const int row = rowA + 16 * a;
                const bf16x8 afr = lds_read<bf16x8>(As, row * 64 + 16 * (q ^ s64));
                const int idx = lds_read<uint16_t>(Ms, row * 8 + 2 * q);
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    acc[a][b] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(afr, bfr[b], acc[a][b],
                                                                          idx, 0, 0);
            }
        } else {
            const char* As = cur;
            const char* Bs = cur + C::A_BYTES;
            bf16x8 bfr[8];
#pragma unroll
            for (int b = 0; b < 8; ++b)
                bfr[b] = lds_read<bf16x8>(Bs, (rowB + 16 * b) * 64 + 16 * (q ^ s64));
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const bf16x8 afr = lds_read<bf16x8>(As, (rowA + 16 * a) * 64 + 16 * (q ^ s64));
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[b], acc[a][b], 0,
                                                                        0, 0);
            }
        }
        if (t + 1 < nk) {
            // wait for stage t+1; the stages issued after it may stay in flight
            const int later = min(nk - 2 - t, C::NSTAGE - 2);
            if (later == C::NSTAGE - 2) {
                wait_vmcnt<(C::NSTAGE - 2) * C::DMA_PER_STAGE>();
            } else if (C::NSTAGE == 4 && later == 1) {
                wait_vmcnt<C::DMA_PER_STAGE>();
            } else {
                __builtin_amdgcn_s_waitcnt(0);
            }
            block_barrier();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // all waves done with the ring before LDS is reused

    // ---- LoRA up-projection: acc += (T / s) LA^T  ----------------------------
    if constexpr (SPARSE) {
        if (R > 0) {
            // T / s (rows m0..) and LA (rows n0..), 256 x 64 bf16 each, zero past
            // R, in swizzled 128-byte rows.  All loads are issued before any is
            // used (clamped in-bounds addresses; out-of-range chunks are zeroed).
            char* Ts = smem;
            char* Ls = smem + 32 * 1024;
            const float* s_lds = reinterpret_cast<const float*>(smem + C::SCALE_OFF);
            u32x4 traw[8], lraw[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = tid + NT * j;
                const int row = c >> 3, kc = min(8 * (c & 7), R - 8);
                traw[j] = *reinterpret_cast<const u32x4*>(T + size_t(min(m0 + row, M - 1)) * R + kc);
                lraw[j] = *reinterpret_cast<const u32x4*>(LA + size_t(min(n0 + row, N - 1)) * R + kc);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = tid + NT * j;
                const int row = c >> 3, ch = c & 7;
                const int off = row * 128 + 16 * (ch ^ swz128(row));
                const bool live = 8 * ch < R;
                const float inv = 1.0f / s_lds[row];
                const u32x4 raw = traw[j];
                u32x4 tv;
                tv.x = pack_bf16x2(bf16_lo(raw.x) * inv, bf16_hi(raw.x) * inv);
                tv.y = pack_bf16x2(bf16_lo(raw.y) * inv, bf16_hi(raw.y) * inv);
                tv.z = pack_bf16x2(bf16_lo(raw.z) * inv, bf16_hi(raw.z) * inv);
                tv.w = pack_bf16x2(bf16_lo(raw.w) * inv, bf16_hi(raw.w) * inv);
                const u32x4 zero = {0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(Ts + off) = live ? tv : zero;
                *reinterpret_cast<u32x4*>(Ls + off) = live ? lraw[j] : zero;
            }
            __syncthreads();
            for (int ks = 0; ks < (R + 31) / 32; ++ks) {
                bf16x8 bfr[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    bfr[b] = lds_read<bf16x8>(Ls, (rowB + 16 * b) * 128 + 16 * ((4 * ks + q) ^ s128));
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    const bf16x8 afr =
                        lds_read<bf16x8>(Ts, (rowA + 16 * a) * 128 + 16 * ((4 * ks + q) ^ s128));
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[b], acc[a][b],
                                                                            0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: y = s * acc (sparse) or acc (dense), bf16, via LDS --------
    char* ep = smem + C::EPI_OFF + wave * 4096;  // 16 rows x 128 cols bf16
    const bool vec_ok = (N & 7) == 0;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const int row_l = 16 * a + 4 * q;  // row within the wave tile of element e = 0
        f32x4 s4 = {1.f, 1.f, 1.f, 1.f};
        if constexpr (SPARSE)
            s4 = *reinterpret_cast<const f32x4*>(smem + C::SCALE_OFF + 4 * (wm * 128 + row_l));
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                *reinterpret_cast<uint16_t*>(ep + (4 * q + e) * 256 + (16 * b + r) * 2) =
                    __builtin_bit_cast(uint16_t, static_cast<__bf16>(s4[e] * acc[a][b][e]));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane -> row lane/4 of the 16, 32 columns starting at (lane%4)*32
        const int orow = m0 + wm * 128 + 16 * a + (lane >> 2);
        const int ocol = n0 + wn * 128 + (lane & 3) * 32;
        if (orow < M) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 v = lds_read<u32x4>(ep, (lane >> 2) * 256 + (lane & 3) * 64 + 16 * i);
                const int col = ocol + 8 * i;
                uint16_t* dst = Y + size_t(orow) * size_t(N) + col;
                if (vec_ok && col + 8 <= N) {
                    *reinterpret_cast<u32x4*>(dst) = v;
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int h = 0; h < 8; ++h)
                        if (col + h < N) dst[h] = uint16_t(w[h >> 1] >> (16 * (h & 1)));
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

lynx_status launch_gemm_sparse_tiled(const uint16_t* values, const uint8_t* meta,
                                     const float* scale, const uint16_t* T, const uint16_t* W,
                                     const uint16_t* LA, uint16_t* Y, int M, int N, int K, int R,
                                     hipStream_t stream) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_tiled<true>, dim3(tiles), dim3(NT), 0, stream, values, meta, scale, T,
                       W, LA, Y, M, N, K, R);
    return launch_status();
}

lynx_status launch_gemm_dense_tiled(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M,
                                    int N, int K, hipStream_t stream) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_tiled<false>, dim3(tiles), dim3(NT), 0, stream, X, nullptr, nullptr,
                       nullptr, W, nullptr, Y, M, N, K, 0);
    return launch_status();
}

}  // namespace lynx
