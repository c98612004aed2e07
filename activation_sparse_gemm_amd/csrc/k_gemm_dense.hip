// Tiled dense GEMM for gfx950: K3 (dense bf16 MFMA, gemm_dense32), the
// dense layer Y = X W^T that the sparse layer's speedup is quoted against
// (RT-Lynx page, 주요 결과, speed item: "Dense 대비").  It is built like the
// sparse GEMM of k_gemm.hip (persistent 256 x 256 or 256 x 192 tiles, 4
// waves of 128 x 128, LDS-DMA ring running across tiles, XCD-aware tile
// order, direct-store epilogue); the shared helpers are in lynx_tile.h.
#include <type_traits>

#include "lynx_tile.h"

namespace lynx {
namespace {

// ---------------------------------------------------------------------------
// K3: dense bf16 GEMM Y = X W^T with v_mfma_f32_32x32x16_bf16, built like K2.
//
// Persistent workgroups of 4 waves walk 256 x 256 tiles; each wave's 128 x 128
// is 4 x 4 accumulator tiles of 32 x 32.  Stages of 32 channels (X and W
// 256 x 64 B each, swizzled 64-byte rows, 32 KB) in a ring of 4 slots; a
// stage is two 16-channel sub-steps of 16 MFMAs (32 cycles each, 1024 per
// stage as in K2, with 32 KB instead of 50 KB to move).  Stage u's 8 DMA
// instructions go out in two halves, the first in stage u - 4's sub-step 1
// right after the barrier that frees slot u % 4, the second in stage u - 3's
// sub-step 0.  The ring runs on across tiles: the stages after a tile's last
// one are the next tile's first four, in flight during the epilogue.  Lane
// l, r = l % 32, h = l / 32 (pinned by the probe tests): A = row r, B =
// column r, channels 8h .. 8h+7 of the 16-channel sub-step (16-byte chunk
// 2 sub + h of the 64-byte LDS row); D as in K2.
// ---------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(NT, 1) void gemm_dense32(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ W,
                                                       uint16_t* __restrict__ Y, int M, int N,
                                                       int K) {
    constexpr int TN = 64 * NB;                    // tile columns (256 or 192)
    constexpr int WC = 32 * NB;                    // columns per wave
    constexpr int kS = 4 * NB;                     // MFMAs per sub-step
    constexpr int kReads = 4 + NB;                 // LDS reads per fragment set
    constexpr int kRow = 64;                       // LDS bytes per row per stage
    constexpr int kABytes = BM * kRow, kBBytes = TN * kRow;
    constexpr int kStage = kABytes + kBBytes;      // 32 KB (28 KB at NB = 3)
    constexpr int kSlots = 4;
    constexpr int kDmaA = kABytes / 1024 / 4, kDmaB = kBBytes / 1024 / 4;  // per wave
    constexpr int kDma = kDmaA + kDmaB;            // 8 (7) per wave and stage
    constexpr int kH0 = (kDma + 1) / 2, kH1 = kDma - kH0;  // the two halves of a stage's DMA
    static_assert(kReads + kH1 <= kS && kReads <= kS - 4 && kH0 <= kS - 4, "stage slots");
    constexpr int kEpiOff = kSlots * kStage;
    constexpr int kEpiWave = 8 * 256;
    constexpr int kLds = kEpiOff + 4 * kEpiWave;
    static_assert(kLds <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, h = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + TN - 1) / TN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = K / 32;  // >= 4: the dispatcher sends K = 64 to the 64 x 64 kernel

    // instruction j of wave w moves rows 16 (w + 4j) + l/4 of a 256-row operand
    // (64-byte LDS rows); lane l lands at byte 16 l of the instruction's 1 KB,
    // its source is the chunk the row's swizzle puts there
    const uint32_t lds0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
    const i32x4 rsA = make_rsrc(X, uint32_t(M) * uint32_t(2 * K));
    const i32x4 rsB = make_rsrc(W, uint32_t(N) * uint32_t(2 * K));
    uint32_t voffA[kDmaA], voffB[kDmaB];  // current tile
    auto offsets = [&](int tm0, int tn0, uint32_t* oa, uint32_t* ob) {
        const int l = fresh_lane();
#pragma unroll
        for (int j = 0; j < kDmaA; ++j) {
            const int row = 16 * (wave + 4 * j) + (l >> 2), ph = l & 3;
            oa[j] = uint32_t(tm0 + row) * uint32_t(2 * K) + uint32_t(16 * (ph ^ swz64(row)));
        }
#pragma unroll
        for (int j = 0; j < kDmaB; ++j) {
            const int row = 16 * (wave + 4 * j) + (l >> 2), ph = l & 3;
            ob[j] = uint32_t(tn0 + row) * uint32_t(2 * K) + uint32_t(16 * (ph ^ swz64(row)));
        }
    };
    // DMA instruction k (0..7) of stage t (of the tile whose offsets are oa/ob)
    auto dma = [&](const uint32_t* oa, const uint32_t* ob, int t, int soff, int k) {
        const uint32_t base = lds0 + uint32_t(soff);
        if (k < kDmaA) {
            dma16(base + 1024 * (wave + 4 * k), oa[k], rsA, uint32_t(t * kRow));
        } else {
            const int j = k - kDmaA;
            dma16(base + kABytes + 1024 * (wave + 4 * j), ob[j], rsB, uint32_t(t * kRow));
        }
    };

    const int s64 = swz64(r);
    const int offA = (wm * 128 + r) * kRow;   // + a * 2048
    const int offB = (wn * WC + r) * kRow;    // + b * 2048
    struct Frags {
        bf16x8 a[4], b[NB];
    };
    Frags fr[2];
    // read n (0..kReads-1) of a set: A0, B0, A1, A2, A3, B1, B2 (, B3):
    // consumption order
    auto read_n = [&](int soff, int sub, Frags& f, int n) {
        constexpr int isb[8] = {0, 1, 0, 0, 0, 1, 1, 1};
        constexpr int blk[8] = {0, 0, 1, 2, 3, 1, 2, 3};
        const char* As = smem + soff;
        const int c = 16 * ((2 * sub + h) ^ s64);
        if (isb[n]) {
            f.b[blk[n]] = lds_read<bf16x8>(As + kABytes, offB + blk[n] * 2048 + c);
        } else {
            f.a[blk[n]] = lds_read<bf16x8>(As, offA + blk[n] * 2048 + c);
        }
    };
    f32x16 acc[4][NB];
    auto mma = [&](const Frags& f, int k) {
        const int a = k & 3, b = k >> 2;
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[a], f.b[b], acc[a][b], 0, 0, 0);
    };

    bool has_next = false;
    int m0n = 0, n0n = 0;
    // instruction i of half `half` of stage u: of this tile if u < nk, else of
    // the next tile (stage u - nk; nothing after the last tile).  The next
    // tile's offsets are formed on the fly: this only runs in the last stages.
    auto dma_u = [&](auto main_c, int u, int soff, int half, int i) {
        constexpr bool MAIN = decltype(main_c)::value;
        const int k = half * kH0 + i;
        if (MAIN || u < nk) {
            dma(voffA, voffB, u, soff, k);
        } else if (has_next) {
            const int j = k < kDmaA ? k : k - kDmaA;
            const int l = fresh_lane();
            const int row = 16 * (wave + 4 * j) + (l >> 2), ph = l & 3;
            const uint32_t off = uint32_t((k < kDmaA ? m0n : n0n) + row) * uint32_t(2 * K) +
                                 uint32_t(16 * (ph ^ swz64(row)));
            dma16(lds0 + uint32_t(soff) + (k < kDmaA ? 0 : kABytes) + 1024 * (wave + 4 * j), off,
                  k < kDmaA ? rsA : rsB, uint32_t((u - nk) * kRow));
        }
    };

    int sl[kSlots] = {0, kStage, 2 * kStage, 3 * kStage};  // slots of stages t .. t+3
    // one stage; MAIN: every load it issues belongs to this tile (t + 4 < nk);
    // WAIT = DMA instructions issued after stage t + 1's last
    auto stage = [&](int t, auto main_c, int wait) {
#pragma unroll
        for (int k = 0; k < kS; ++k) {
            mma(fr[0], k);
            if (k < kReads) read_n(sl[0], 1, fr[1], k);
            if (k >= kReads && k - kReads < kH1) dma_u(main_c, t + 3, sl[3], 1, k - kReads);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mma(fr[1], k);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (wait >= 2 * kDma) {
            wait_vmcnt_lgkm0<2 * kDma>();
        } else if (wait >= kDma) {
            wait_vmcnt_lgkm0<kDma>();
        } else {
            wait_vmcnt_lgkm0<0>();
        }
        block_barrier();
#pragma unroll
        for (int k = 4; k < kS; ++k) {
            mma(fr[1], k);
            if (k - 4 < kReads) read_n(sl[1], 0, fr[0], k - 4);
            if (k - 4 < kH0) dma_u(main_c, t + 4, sl[0], 0, k - 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int freed = sl[0];
        sl[0] = sl[1];
        sl[1] = sl[2];
        sl[2] = sl[3];
        sl[3] = freed;
    };

    const bool vec_ok = (N & 7) == 0;
    const __amdgpu_buffer_rsrc_t rsY =
        __builtin_amdgcn_make_buffer_rsrc(Y, 0, int(uint32_t(M) * uint32_t(N) * 2u), kRsrcWord3);
    char* ep = smem + kEpiOff + wave * kEpiWave;

    int v = blockIdx.x;
    int m0, n0;
    {
        int tm, tn;
        tile_of(v, tiles_m, tiles_n, tm, tn);
        m0 = tm * BM;
        n0 = tn * TN;
    }
    offsets(m0, n0, voffA, voffB);
    __builtin_amdgcn_s_waitcnt(0);
    // first tile: stages 0, 1, 2 and the first half of 3
    for (int t = 0; t < 3; ++t)
        for (int k = 0; k < kDma; ++k) dma(voffA, voffB, t, sl[t], k);
    for (int i = 0; i < kH0; ++i) dma(voffA, voffB, 3, sl[3], i);

    for (; v < ntiles; v += gridDim.x) {
        // stages 0..2 and half of 3 of this tile are in flight
        const int vn = v + gridDim.x;
        has_next = vn < ntiles;
        m0n = m0;
        n0n = n0;
        if (has_next) {
            int tm, tn;
            tile_of(vn, tiles_m, tiles_n, tm, tn);
            m0n = tm * BM;
            n0n = tn * TN;
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[a][b] = f32x16{};
        wait_vmcnt<2 * kDma + kH0>();  // stage 0 has landed
        block_barrier();
#pragma unroll
        for (int n = 0; n < kReads; ++n) read_n(sl[0], 0, fr[0], n);

        const int nx = has_next ? kDma : 0;  // DMA instructions of a next-tile stage
        for (int t = 0; t < nk - 4; ++t) stage(t, std::true_type{}, 2 * kDma);
        // stage t + 1's later loads: stages t + 2 and t + 3, of this tile or the next
        for (int t = nk - 4; t < nk; ++t)
            stage(t, std::false_type{}, (t + 2 < nk ? kDma : nx) + (t + 3 < nk ? kDma : nx));

        // ---- epilogue: as in K2 (interior tiles direct, edge tiles staged)
        if (vec_ok && n0 + TN <= N) {
            store_block_direct<NB>(acc, rsY, N, m0 + wm * 128, n0 + wn * WC);
        } else {
            // ---- epilogue: y = acc, bf16, 8 rows at a time through LDS ----------
            // (the same staging as K2's epilogue, scale 1)
    #pragma unroll
            for (int a = 0; a < 4; ++a) {
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rbase = wm * 128 + 32 * a + 8 * j;
    #pragma unroll
                    for (int b = 0; b < NB; ++b)
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int lr = 4 * h + i;
                            *reinterpret_cast<uint16_t*>(ep + lr * 256 + (((32 * b + r) * 2) ^ (h << 7))) =
                                __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[a][b][4 * j + i]));
                        }
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    const int el = fresh_lane();
                    const int srow = el >> 3;
                    const int orow = m0 + rbase + srow;
                    const int ocol = n0 + wn * WC + (el & 7) * 16;
                    if (orow < M && (el & 7) < 2 * NB) {
                        const int sb = srow * 256 + (((el & 7) * 32) ^ ((srow >> 2) << 7));
    #pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const u32x4 w4 = lds_read<u32x4>(ep, sb + 16 * i);
                            const int col = ocol + 8 * i;
                            const uint32_t yoff = (uint32_t(orow) * uint32_t(N) + uint32_t(col)) * 2u;
                            if (vec_ok && col + 8 <= N) {
                                __builtin_amdgcn_raw_buffer_store_b128(w4, rsY, yoff, 0, 0);
                            } else {
                                const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
    #pragma unroll
                                for (int q2 = 0; q2 < 8; ++q2)
                                    if (col + q2 < N)
                                        __builtin_amdgcn_raw_buffer_store_b16(
                                            uint16_t(w[q2 >> 1] >> (16 * (q2 & 1))), rsY,
                                            yoff + 2u * q2, 0, 0);
                            }
                        }
                    }
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
            }
        }
        // the next tile's stages 0..2 and half of 3 are in sl[0..3]
        m0 = m0n;
        n0 = n0n;
        offsets(m0, n0, voffA, voffB);
    }
}

}  // namespace

lynx_status launch_gemm_dense_tiled(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M,
                                    int N, int K, hipStream_t stream) {
    // persistent, with the same choice of tile width as the sparse kernel
    int cus = 0;
    if (device_cu_count(&cus) != LYNX_OK) return LYNX_ERR_DEVICE;
    const long tm = (M + BM - 1) / BM;
    auto tiles_for = [&](int tn) { return tm * ((N + tn - 1) / tn); };
    auto cost = [&](int tn) { return (tiles_for(tn) + cus - 1) / cus * tn; };
    const bool narrow = cost(192) < cost(256);
    const long tiles = tiles_for(narrow ? 192 : 256);
    const int grid = int(tiles < cus ? tiles : cus);
    if (narrow) {
        hipLaunchKernelGGL(gemm_dense32<3>, dim3(grid), dim3(NT), 0, stream, X, W, Y, M, N, K);
    } else {
        hipLaunchKernelGGL(gemm_dense32<4>, dim3(grid), dim3(NT), 0, stream, X, W, Y, M, N, K);
    }
    return launch_status();
}

}  // namespace lynx
