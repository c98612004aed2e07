// Measurement prototype, not part of liblynx: the 2:4 sparse GEMM with the
// sparsifier inside its operand load, the single execution path the RT-Lynx
// page describes (핵심 기여, third item: pattern decision, Top-K and
// compression in one path; 기술 상세: the 2:4 activation formed directly in
// registers).  It exists to measure that design against the library's
// sparsifier + sparse GEMM pair on gfx950; the library does not use it.
//
// Built like the dense GEMM of the library (persistent 256 x 256 / 256 x 192
// tiles, 4 waves of 128 x 128, 32-channel stages of dense X and W through a
// 4-slot LDS-DMA ring), but each wave reads 16 dense channels of its rows per
// lane and selects the top 2 of every 4 in registers (the same integer key as
// the library's sparsifier: |x| bits and the position, ties to the lower
// index), accumulates the row norms along K, feeds the kept values and index
// word to v_smfmac_f32_32x32x32_bf16, and scales each row by
// s = ||x|| / ||x~|| before the store.  Left out, as a prototype: the LoRA
// term, the exact fp64 norm pass for extreme rows, and tiles with columns
// past N (the measured shapes have none).
//
// Entry point (C ABI, device pointers, bf16 as uint16_t):
//   proto_gemm_fused(X [M][K], W [N][K], Y [M][N], M, N, K, stream) -> 0, or
//   2 for a shape outside what it handles (K % 128, N % 192 / 256, M % 256).
#include <type_traits>

#include "lynx_tile.h"

namespace lynx {
namespace {

// Prototype (measurement only): the sparse GEMM with the sparsifier inside its
// operand load.  Dense X comes through the same LDS ring as the dense kernel
// (32-channel stages); each wave selects the top 2 of 4 of its A fragment in
// registers (16 dense channels per lane -> 8 kept values + index word),
// accumulates the row norms along K, and scales the rows by s at the end.
// No LoRA term, no exact pass for extreme rows.
__device__ __forceinline__ uint32_t sel2(uint32_t lo, uint32_t hi, uint32_t& kept) {
    const uint32_t k0 = ((lo & 0x7FFFu) << 2) | 3u;
    const uint32_t k1 = ((lo >> 14) & 0x1FFFCu) | 2u;
    const uint32_t k2 = ((hi & 0x7FFFu) << 2) | 1u;
    const uint32_t k3 = (hi >> 14) & 0x1FFFCu;
    const uint32_t hi01 = max(k0, k1), lo01 = min(k0, k1);
    const uint32_t hi23 = max(k2, k3), lo23 = min(k2, k3);
    const uint32_t second = max(min(hi01, hi23), max(lo01, lo23));
    const uint32_t m = (k0 >= second ? 1u : 0u) | (k1 >= second ? 2u : 0u) |
                       (k2 >= second ? 4u : 0u) | (k3 >= second ? 8u : 0u);
    const uint32_t i0 = __builtin_ctz(m);
    const uint32_t i1 = 31u - __builtin_clz(m);
    const uint32_t sel = 0x01000100u + i0 * 0x0202u + i1 * 0x02020000u;
    kept = __builtin_amdgcn_perm(hi, lo, sel);
    return i0 | (i1 << 2);
}
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float d2(uint32_t w, float acc) {
    const bf16x2v v = __builtin_bit_cast(bf16x2v, w);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

template <int NB>
__global__ __launch_bounds__(NT, 1) void gemm_fused32(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ W,
                                                       uint16_t* __restrict__ Y, int M, int N,
                                                       int K) {
    constexpr int TN = 64 * NB, WC = 32 * NB, kS = 4 * NB;
    constexpr int kRow = 64;
    constexpr int kABytes = BM * kRow, kBBytes = TN * kRow;
    constexpr int kStage = kABytes + kBBytes;
    constexpr int kSlots = 4;
    constexpr int kDmaA = kABytes / 1024 / 4, kDmaB = kBBytes / 1024 / 4;
    constexpr int kDma = kDmaA + kDmaB;
    constexpr int kSOff = kSlots * kStage;   // s of the tile's 256 rows
    constexpr int kLds = kSOff + BM * 4;
    static_assert(kLds <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    float* s_lds = reinterpret_cast<float*>(smem + kSOff);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, h = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + TN - 1) / TN;
    const int ntiles = tiles_m * tiles_n;
    const int nk = K / 32;
    const uint32_t lds0 = lds_addr(smem);
    const i32x4 rsA = make_rsrc(X, uint32_t(M) * uint32_t(2 * K));
    const i32x4 rsB = make_rsrc(W, uint32_t(N) * uint32_t(2 * K));
    uint32_t voffA[kDmaA], voffB[kDmaB];
    auto offsets = [&](int tm0, int tn0) {
        const int l = fresh_lane();
#pragma unroll
        for (int j = 0; j < kDmaA; ++j) {
            const int row = 16 * (wave + 4 * j) + (l >> 2), ph = l & 3;
            voffA[j] = uint32_t(tm0 + row) * uint32_t(2 * K) + uint32_t(16 * (ph ^ swz64(row)));
        }
#pragma unroll
        for (int j = 0; j < kDmaB; ++j) {
            const int row = 16 * (wave + 4 * j) + (l >> 2), ph = l & 3;
            voffB[j] = uint32_t(tn0 + row) * uint32_t(2 * K) + uint32_t(16 * (ph ^ swz64(row)));
        }
    };
    // all DMAs of stage t into slot soff (stages past K read out of range)
    auto dma_stage = [&](int t, int soff) {
        const uint32_t base = lds0 + uint32_t(soff);
        const uint32_t so = t < nk ? uint32_t(t * kRow) : 0u;
#pragma unroll
        for (int k = 0; k < kDmaA; ++k)
            dma16(base + 1024 * (wave + 4 * k), t < nk ? voffA[k] : 0xFFFFFFF0u, rsA, so);
#pragma unroll
        for (int j = 0; j < kDmaB; ++j)
            dma16(base + kABytes + 1024 * (wave + 4 * j), t < nk ? voffB[j] : 0xFFFFFFF0u, rsB, so);
    };
    const int s64 = swz64(r);
    const int offA = (wm * 128 + r) * kRow, offB = (wn * WC + r) * kRow;
    struct Raw { u32x4 a[4][2]; bf16x16 b[NB]; };
    struct Sel { bf16x8 v[4]; int i[4]; };
    Raw raw[2];
    Sel sel;
    double n2[4], nt2[4];
    // lane (r, h): A = row r, dense channels [16 h, 16 h + 16) = chunks 2 h, 2 h + 1;
    // B = column r, channels [8 h, 8 h + 8) and [16 + 8 h, 24 + 8 h) = chunks h, 2 + h
    auto read_all = [&](int soff, Raw& f) {
        const char* As = smem + soff;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f.a[a][0] = lds_read<u32x4>(As, offA + a * 2048 + 16 * ((2 * h) ^ s64));
            f.a[a][1] = lds_read<u32x4>(As, offA + a * 2048 + 16 * ((2 * h + 1) ^ s64));
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const bf16x8 lo = lds_read<bf16x8>(As + kABytes, offB + b * 2048 + 16 * (h ^ s64));
            const bf16x8 hi = lds_read<bf16x8>(As + kABytes, offB + b * 2048 + 16 * ((2 + h) ^ s64));
            f.b[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        }
    };
    auto select_a = [&](const Raw& f, int a) {
        uint32_t kp[4];
        int code = 0;
        float pn = 0.f, pt = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4 x = f.a[a][c];
            pn = d2(x.x, pn); pn = d2(x.y, pn); pn = d2(x.z, pn); pn = d2(x.w, pn);
            code |= int(sel2(x.x, x.y, kp[2 * c]) << (8 * c));
            code |= int(sel2(x.z, x.w, kp[2 * c + 1]) << (8 * c + 4));
        }
        pt = d2(kp[0], pt); pt = d2(kp[1], pt); pt = d2(kp[2], pt); pt = d2(kp[3], pt);
        n2[a] += double(pn);
        nt2[a] += double(pt);
        sel.v[a] = __builtin_bit_cast(bf16x8, u32x4{kp[0], kp[1], kp[2], kp[3]});
        sel.i[a] = code;
    };
    f32x16 acc[4][NB];
    int sl[kSlots] = {0, kStage, 2 * kStage, 3 * kStage};
    const bool vec_ok = (N & 7) == 0;
    const __amdgpu_buffer_rsrc_t rsY =
        __builtin_amdgcn_make_buffer_rsrc(Y, 0, int(uint32_t(M) * uint32_t(N) * 2u), kRsrcWord3);
    for (int v = blockIdx.x; v < ntiles; v += gridDim.x) {
        int tm, tn;
        tile_of(v, tiles_m, tiles_n, tm, tn);
        const int m0 = tm * BM, n0 = tn * TN;
        offsets(m0, n0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            n2[a] = nt2[a] = 0.0;
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[a][b] = f32x16{};
        }
        for (int t = 0; t < 4; ++t) dma_stage(t, sl[t]);
        wait_vmcnt_lgkm0<3 * kDma>();
        block_barrier();
        read_all(sl[0], raw[0]);
        wait_lgkm0();
#pragma unroll
        for (int a = 0; a < 4; ++a) select_a(raw[0], a);
        // stage t: sel + raw[t & 1].b hold stage t; the reads of stage t + 1
        // go out after the barrier, its selection after the last SMFMACs
        auto stage = [&](int t, Raw& cur, Raw& nxt) {
#pragma unroll
            for (int k = 0; k < kS; ++k) {
                const int a = k & 3, b = k >> 2;
                acc[a][b] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(sel.v[a], cur.b[b], acc[a][b],
                                                                      sel.i[a], 0, 0);
                if (k == 1) {
                    wait_vmcnt_lgkm0<2 * kDma>();   // stage t + 1 landed (own)
                    block_barrier();                // ... for every wave; slot of t is free
                    read_all(sl[1], nxt);
                    dma_stage(t + 4, sl[0]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_lgkm0();
#pragma unroll
            for (int a = 0; a < 4; ++a) select_a(nxt, a);
            const int fr = sl[0];
            sl[0] = sl[1]; sl[1] = sl[2]; sl[2] = sl[3]; sl[3] = fr;
        };
        for (int t = 0; t < nk; t += 2) {
            stage(t, raw[0], raw[1]);
            stage(t + 1, raw[1], raw[0]);
        }
        // s per row: lanes (r, 0) and (r, 1) hold the two halves of row r
        if (wn == 0) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                double x = n2[a] + __shfl_xor(n2[a], 32), y = nt2[a] + __shfl_xor(nt2[a], 32);
                if (h == 0) s_lds[wm * 128 + 32 * a + r] = y > 0.0 ? float(sqrt(x / y)) : 1.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 sv = *reinterpret_cast<const f32x4*>(s_lds + wm * 128 + 32 * a + 8 * j + 4 * h);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[a][b][4 * j + i] *= sv[i];
            }
        if (vec_ok && n0 + TN <= N) store_block_direct<NB>(acc, rsY, N, m0 + wm * 128, n0 + wn * WC);
    }
}
}  // namespace
}  // namespace lynx

using namespace lynx;

extern "C" int proto_gemm_fused(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                                int64_t N, int64_t K, void* stream) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || M % 256 != 0) return 2;
    if ((M + 256) * K >= (int64_t(1) << 31) || (N + 256) * K >= (int64_t(1) << 31) ||
        (M + 256) * N >= (int64_t(1) << 31))
        return 2;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 5;
    const long tm = M / BM;
    auto tiles_for = [&](int tn) { return tm * ((N + tn - 1) / tn); };
    auto cost = [&](int tn) { return (tiles_for(tn) + cus - 1) / cus * tn; };
    const bool narrow = cost(192) < cost(256);
    if (N % (narrow ? 192 : 256) != 0) return 2;
    const long tiles = tiles_for(narrow ? 192 : 256);
    const int grid = int(tiles < cus ? tiles : cus);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (narrow) {
        hipLaunchKernelGGL(gemm_fused32<3>, dim3(grid), dim3(NT), 0, s, X, W, Y, int(M), int(N), int(K));
    } else {
        hipLaunchKernelGGL(gemm_fused32<4>, dim3(grid), dim3(NT), 0, s, X, W, Y, int(M), int(N), int(K));
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
