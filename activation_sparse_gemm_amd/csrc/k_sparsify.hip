// K1: online 2:4 activation sparsification fused with the LoRA down-projection.
//
// RT-Lynx page (aitrends.kr), 방법론 "핵심 메커니즘": Top-K 2:4 selection of the
// activation, S(X) = s X~, and the 2:4 activation handed to the sparse GEMM in
// the sparse unit's operand format; 핵심 기여, third item: pattern decision,
// Top-K and compression done in one execution path; 코드 예제: s = ||X||/||X~||.
// The LoRA branch reads the same dense X (Yr = X (LA LB)^T), so T = X LB^T is
// formed here from the registers that already hold X.
//
// Work decomposition (one read of X):
//   workgroup = ROWT row tiles of 16 rows (tokens) x all of K; its NW waves
//   split K in 128-channel chunks (the last one 64 channels wide when
//   K % 128 == 64).  Lane l: row r = l % 16 of every row tile, quarter
//   q = l / 16; in chunk c it owns channels [128c + 32q, 128c + 32q + 32) of
//   each of its ROWT rows: 8 groups of 4 per row, loaded as 4 x 16 bytes.
//   Lanes whose channels lie past K (quarters 2 and 3 of a 64-wide last chunk)
//   load nothing, hold zeros (which add nothing to the norms or T) and store
//   nothing; those checks are compiled only into the instantiation for
//   K % 128 == 64 (HALF), so the loop for K % 128 == 0 carries none of them.
//   - selection + packing in registers: 16 kept values (32 B) and 8 codes (4 B)
//     per row, lane and chunk, stored in the 16-row x 64-channel tile order of
//     the packed operand (a row tile is exactly one tile row-block; rows past M
//     in the last existing tile are written as zero values and codes (0,1));
//   - row norms ||x||^2 and ||x~||^2 with v_dot2_f32_bf16 (products of bf16 are
//     exact in fp32), summed per chunk in fp32 then in fp64;
//   - T: the lane's 32 channels are the A operand of 4 v_mfma_f32_16x16x32_bf16
//     steps (k-block q of each step), LB rows supply the B operand with the same
//     channel map, one 16-column tile of T per 16 ranks.  Each LB fragment is
//     read from the LDS once and used for all ROWT row tiles, so the LB bytes a
//     workgroup streams from L2 serve 16 ROWT rows.
//   The launcher takes one row tile per workgroup (8 waves) while one round of
//   workgroups covers M, else 2 or 3 row tiles (4 waves, to keep the rows'
//   registers): at M = 9216 three 16-row rounds become one 48-row round.
//   Partial norms and T are reduced across waves through LDS in a fixed order
//   (deterministic), then s and bf16 T are written.
//   Squares of bf16 values are exact in fp32 only while they neither overflow
//   nor underflow; a row whose ||x||^2 from the fast path is outside
//   [2^-60, 2^100] (or is not finite, or is zero) is recomputed exactly: one
//   wave re-reads the row, decodes bf16 to fp64 with integer operations and
//   sums the squares in fp64.  Rows inside that range lose at most 2^-52 of
//   ||x||^2 to flushed tiny terms.
#include "lynx_internal.h"

namespace lynx {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = 16;
constexpr int kChunk = 128;

// Top-2 of one group of 4 bf16 values given as lo = x0 | x1 << 16 and
// hi = x2 | x3 << 16.  Returns the 4-bit code i0 | i1 << 2 (i0 < i1) and, in
// `kept`, the pair x_i0 | x_i1 << 16 (bit-exact copies).
// Ordering key: |x| (the bf16 bits without sign, exact for finite values, and
// -0 == +0) times 4 plus (3 - j), so all keys differ, a larger |x| wins and an
// equal |x| goes to the lower index j.
__device__ __forceinline__ uint32_t select_group(uint32_t lo, uint32_t hi, uint32_t& kept) {
    const uint32_t k0 = ((lo & 0x7FFFu) << 2) | 3u;
    const uint32_t k1 = ((lo >> 14) & 0x1FFFCu) | 2u;
    const uint32_t k2 = ((hi & 0x7FFFu) << 2) | 1u;
    const uint32_t k3 = (hi >> 14) & 0x1FFFCu;
    const uint32_t hi01 = max(k0, k1), lo01 = min(k0, k1);
    const uint32_t hi23 = max(k2, k3), lo23 = min(k2, k3);
    // second largest of four distinct keys
    const uint32_t second = max(min(hi01, hi23), max(lo01, lo23));
    const uint32_t m = (k0 >= second ? 1u : 0u) | (k1 >= second ? 2u : 0u) |
                       (k2 >= second ? 4u : 0u) | (k3 >= second ? 8u : 0u);
    const uint32_t i0 = __builtin_ctz(m);
    const uint32_t i1 = 31u - __builtin_clz(m);
    // v_perm_b32 byte selector: bytes 0..3 of {hi:lo} are lo, 4..7 are hi;
    // element j occupies bytes 2j, 2j+1.
    const uint32_t sel = 0x01000100u + i0 * 0x0202u + i1 * 0x02020000u;
    kept = __builtin_amdgcn_perm(hi, lo, sel);
    return i0 | (i1 << 2);
}

// Exact bf16 -> fp64 from the bit pattern (no dependence on denormal modes).
__device__ __forceinline__ double bf16_to_f64(uint32_t b) {
    const uint32_t e = (b >> 7) & 0xFFu, m = b & 0x7Fu;
    double v;
    if (e == 0) {
        v = double(m) * 0x1p-133;  // subnormal bf16: m * 2^-133
    } else {
        v = __longlong_as_double(static_cast<long long>((uint64_t(e) + 896u) << 52 |
                                                        uint64_t(m) << 45));
    }
    return (b & 0x8000u) ? -v : v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float dot2_self(uint32_t w, float acc) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

// RT = R / 16 column tiles of T (0..4); ROWT row tiles of 16 rows; NW waves;
// HALF: K % 128 == 64 (the last chunk is 64 channels wide)
template <int RT, int ROWT, int NW, bool HALF>
__global__ __launch_bounds__(NW * 64) void sparsify_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ LB, int M, int K,
    uint16_t* __restrict__ values, uint8_t* __restrict__ meta, float* __restrict__ scale,
    uint16_t* __restrict__ T) {
    constexpr int R = RT * 16;
    constexpr int kWgRows = kRows * ROWT;
    __shared__ double red_norm[NW][kWgRows][2];
    __shared__ int exact_row[kWgRows];
    // per-wave LB chunk (R rows x 256 B, XOR-swizzled 16-byte pieces); after
    // the main loop the same memory holds the cross-wave T partials
    constexpr int kLbBytes = RT > 0 ? R * 256 : 64 * ROWT;
    __shared__ __attribute__((aligned(16))) char lbw[NW][kLbBytes];
    static_assert(sizeof(lbw) >= sizeof(float) * NW * kWgRows * (RT > 0 ? R : 1),
                  "T partials fit in the LB staging area");
    float(*red_T)[kWgRows][RT > 0 ? R : 1] =
        reinterpret_cast<float(*)[kWgRows][RT > 0 ? R : 1]>(&lbw[0][0]);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane & 15;
    const int q = lane >> 4;
    const int m0 = blockIdx.x * kWgRows;
    const int nchunks = (K + kChunk - 1) / kChunk;
    const int steps = K / 64;

    const uint16_t* xrow[ROWT];
    bool row_ok[ROWT];
#pragma unroll
    for (int u = 0; u < ROWT; ++u) {
        const int row = m0 + 16 * u + r;
        row_ok[u] = row < M;
        xrow[u] = X + size_t(row_ok[u] ? row : M - 1) * size_t(K);
    }
    // packed operand, tile order: tile (block b, 64-channel step s) holds 16 rows
    // x 32 values (1 KB) and 16 rows x 8 meta bytes (128 B); row tile u of this
    // workgroup is block ROWT * blockIdx.x + u
    uint16_t* vtile = values + size_t(blockIdx.x) * ROWT * size_t(steps) * 512 + r * 32;
    uint8_t* mtile = meta + size_t(blockIdx.x) * ROWT * size_t(steps) * 128 + r * 8;

    f32x4 acc[ROWT][RT > 0 ? RT : 1];
#pragma unroll
    for (int u = 0; u < ROWT; ++u)
#pragma unroll
        for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    double n2[ROWT], nt2[ROWT];
#pragma unroll
    for (int u = 0; u < ROWT; ++u) n2[u] = nt2[u] = 0.0;

    auto load_x = [&](int c, u32x4 (*xd)[4]) {
        const int k = c * kChunk + q * 32;
        // K % 64 == 0: a lane's 32 channels are all in range or all past K
        const bool live = !HALF || k < K;
#pragma unroll
        for (int u = 0; u < ROWT; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xd[u][i] = live ? *reinterpret_cast<const u32x4*>(xrow[u] + k + 8 * i)
                                : u32x4{0u, 0u, 0u, 0u};
    };
    auto load_lb = [&](int c, u32x4* ld) {
        const int k = c * kChunk + 8 * (lane & 15);
        const bool live = !HALF || k < K;
#pragma unroll
        for (int j = 0; j < (RT > 0 ? R / 4 : 0); ++j) {
            const int lr = 4 * j + (lane >> 4);
            ld[j] = live ? *reinterpret_cast<const u32x4*>(LB + size_t(lr) * size_t(K) + k)
                         : u32x4{0u, 0u, 0u, 0u};
        }
    };
    u32x4 xv[ROWT][4], lbraw[RT > 0 ? R / 4 : 1];
    if (wave < nchunks) {
        load_x(wave, xv);
        load_lb(wave, lbraw);
    }

    for (int c = wave; c < nchunks; c += nwaves) {
        const int k = c * kChunk + q * 32;
        const bool more = c + nwaves < nchunks;
        u32x4 xn[ROWT][4];
        if (more) load_x(c + nwaves, xn);

#pragma unroll
        for (int u = 0; u < ROWT; ++u) {
            float pn = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pn = dot2_self(xv[u][i].x, pn);
                pn = dot2_self(xv[u][i].y, pn);
                pn = dot2_self(xv[u][i].z, pn);
                pn = dot2_self(xv[u][i].w, pn);
            }
            uint32_t kept[8];
            uint32_t code = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                code |= select_group(xv[u][i].x, xv[u][i].y, kept[2 * i]) << (8 * i);
                code |= select_group(xv[u][i].z, xv[u][i].w, kept[2 * i + 1]) << (8 * i + 4);
            }
            float pt = 0.f;
#pragma unroll
            for (int g = 0; g < 8; ++g) pt = dot2_self(kept[g], pt);
            n2[u] += double(pn);
            nt2[u] += double(pt);

            // channels k .. k+31 = half (q & 1) of step k / 64
            const int step = k >> 6, half = q & 1;
            u32x4* vdst = reinterpret_cast<u32x4*>(vtile + (size_t(u) * steps + step) * 512 + half * 16);
            uint32_t* mdst = reinterpret_cast<uint32_t*>(mtile + (size_t(u) * steps + step) * 128 + half * 4);
            if (HALF && k >= K) {
                // channels past K (64-wide last chunk): nothing to store
            } else if (row_ok[u]) {
                vdst[0] = u32x4{kept[0], kept[1], kept[2], kept[3]};
                vdst[1] = u32x4{kept[4], kept[5], kept[6], kept[7]};
                *mdst = code;
            } else if (m0 + 16 * u < M) {  // padding row of the last (existing) tile
                vdst[0] = u32x4{0u, 0u, 0u, 0u};
                vdst[1] = u32x4{0u, 0u, 0u, 0u};
                *mdst = 0x44444444u;
            }
        }

        // T += X LB^T over these channels; B operand of step i: LB row
        // 16 t + r, channels 32 q + 8 i .. +8 of the chunk, read once from the
        // LDS for all row tiles
        if constexpr (RT > 0) {
            char* lb = lbw[wave];
#pragma unroll
            for (int j = 0; j < R / 4; ++j) {
                const int lr = 4 * j + (lane >> 4);
                *reinterpret_cast<u32x4*>(lb + lr * 256 + 16 * ((lane & 15) ^ (lr & 15))) =
                    lbraw[j];
            }
            if (more) load_lb(c + nwaves, lbraw);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int t = 0; t < RT; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16x8 bv = *reinterpret_cast<const bf16x8*>(
                        lb + (16 * t + r) * 256 + 16 * ((4 * q + i) ^ r));
#pragma unroll
                    for (int u = 0; u < ROWT; ++u)
                        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, xv[u][i]), bv, acc[u][t], 0, 0, 0);
                }
            }
            // the next chunk's writes must not overtake this chunk's reads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < ROWT; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[u][i] = xn[u][i];
        }
    }

    // ---- cross-lane (4 quarters of a row) then cross-wave reductions ----
#pragma unroll
    for (int u = 0; u < ROWT; ++u) {
        double a = n2[u], b = nt2[u];
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        b += __shfl_xor(b, 16);
        b += __shfl_xor(b, 32);
        if (q == 0) {
            red_norm[wave][16 * u + r][0] = a;
            red_norm[wave][16 * u + r][1] = b;
        }
    }
    __syncthreads();  // every wave is done with its LB area before it holds T partials
    // accumulator layout of a 16x16 tile: lane (n = l % 16, q) holds rows 4q..4q+3
#pragma unroll
    for (int u = 0; u < ROWT; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) red_T[wave][16 * u + 4 * q + e][16 * t + r] = acc[u][t][e];
    __syncthreads();

    if (threadIdx.x < kWgRows) {
        const int rr = threadIdx.x;
        double a = 0.0, b = 0.0;
        for (int w = 0; w < nwaves; ++w) {
            a += red_norm[w][rr][0];
            b += red_norm[w][rr][1];
        }
        const bool safe = a >= 0x1p-60 && a <= 0x1p100 && b > 0.0;
        exact_row[rr] = (m0 + rr < M) && !safe;
        if (m0 + rr < M && safe) scale[m0 + rr] = float(sqrt(a / b));
    }
    // T = the waves' partials summed in wave order, four columns per thread
    // (it does not wait for the exact-row decisions above)
    if constexpr (RT > 0) {
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        for (int idx = threadIdx.x; idx < kWgRows * R / 4; idx += blockDim.x) {
            const int rr = idx / (R / 4), c4 = 4 * (idx % (R / 4));
            f32x4 sm = *reinterpret_cast<const f32x4*>(&red_T[0][rr][c4]);
            for (int w = 1; w < nwaves; ++w) sm += *reinterpret_cast<const f32x4*>(&red_T[w][rr][c4]);
            if (m0 + rr < M)
                *reinterpret_cast<u32x2*>(T + size_t(m0 + rr) * R + c4) =
                    __builtin_bit_cast(u32x2, __builtin_convertvector(sm, bf16x4_t));
        }
    }
    __syncthreads();  // exact_row is complete
    // exact fp64 pass for rows outside the fast path's range (rare)
    for (int rr = wave; rr < kWgRows; rr += nwaves) {
        if (!exact_row[rr]) continue;
        const uint32_t* xr = reinterpret_cast<const uint32_t*>(X + size_t(m0 + rr) * size_t(K));
        double a = 0.0, b = 0.0;
        for (int g = lane; g < K / 4; g += 64) {
            const uint32_t lo = xr[2 * g], hi = xr[2 * g + 1];
            uint32_t kept;
            (void)select_group(lo, hi, kept);
            const double x0 = bf16_to_f64(lo & 0xFFFFu), x1 = bf16_to_f64(lo >> 16);
            const double x2 = bf16_to_f64(hi & 0xFFFFu), x3 = bf16_to_f64(hi >> 16);
            const double k0 = bf16_to_f64(kept & 0xFFFFu), k1 = bf16_to_f64(kept >> 16);
            a += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
            b += k0 * k0 + k1 * k1;
        }
        a = wave_sum(a);
        b = wave_sum(b);
        if (lane == 0) scale[m0 + rr] = b > 0.0 ? float(sqrt(a / b)) : 1.0f;
    }
}

// Per-workgroup time of ROWT row tiles (NW = 8 for one tile, 4 for two or
// three), relative to one tile; measured on the MI355X at K = 3072 and 12288,
// R = 64 (µs, K = 3072 / 12288: 16.3 / 52.4, 24.0 / 75.0, 29.7 / 92.1).
constexpr float kRowtCost[4] = {0.f, 1.0f, 1.45f, 1.8f};

template <int RT, bool HALF>
void launch_rt(int rowt, int M, int K, int nchunks, const uint16_t* X, const uint16_t* LB,
               uint16_t* values, uint8_t* meta, float* scale, uint16_t* T, hipStream_t stream) {
    const int nw = rowt == 1 ? 8 : 4;
    const dim3 grid((M + kRows * rowt - 1) / (kRows * rowt)), block(64 * (nchunks < nw ? nchunks : nw));
    if (rowt == 1) {
        hipLaunchKernelGGL((sparsify_kernel<RT, 1, 8, HALF>), grid, block, 0, stream, X, LB, M, K,
                           values, meta, scale, T);
    } else if (rowt == 2) {
        hipLaunchKernelGGL((sparsify_kernel<RT, 2, 4, HALF>), grid, block, 0, stream, X, LB, M, K,
                           values, meta, scale, T);
    } else {
        hipLaunchKernelGGL((sparsify_kernel<RT, 3, 4, HALF>), grid, block, 0, stream, X, LB, M, K,
                           values, meta, scale, T);
    }
}

template <int RT>
void launch_rt(int rowt, int M, int K, int nchunks, const uint16_t* X, const uint16_t* LB,
               uint16_t* values, uint8_t* meta, float* scale, uint16_t* T, hipStream_t stream) {
    if (K % kChunk == 0) {
        launch_rt<RT, false>(rowt, M, K, nchunks, X, LB, values, meta, scale, T, stream);
    } else {
        launch_rt<RT, true>(rowt, M, K, nchunks, X, LB, values, meta, scale, T, stream);
    }
}

}  // namespace

lynx_status launch_sparsify(const uint16_t* X, const uint16_t* LB, int M, int K, int R,
                            uint16_t* values, uint8_t* meta, float* scale, uint16_t* T,
                            hipStream_t stream) {
    const int nchunks = (K + kChunk - 1) / kChunk;
    // Row tiles per workgroup: the fewest rounds of workgroups over the compute
    // units, weighted by the measured cost of a workgroup (one tile when there
    // is no LoRA: nothing is shared between row tiles then).
    int rowt = 1;
    if (R > 0) {
        int cus = 0;
        if (device_cu_count(&cus) != LYNX_OK) return LYNX_ERR_DEVICE;
        const long tiles = (M + kRows - 1) / kRows;
        float best = 0.f;
        for (int t = 1; t <= 3; ++t) {
            const long wgs = (tiles + t - 1) / t;
            const float c = float((wgs + cus - 1) / cus) * kRowtCost[t];
            if (t == 1 || c < best) {
                best = c;
                rowt = t;
            }
        }
    }
    switch (R / 16) {
        case 0:
            launch_rt<0>(1, M, K, nchunks, X, LB, values, meta, scale, T, stream);
            break;
        case 1:
            launch_rt<1>(rowt, M, K, nchunks, X, LB, values, meta, scale, T, stream);
            break;
        case 2:
            launch_rt<2>(rowt, M, K, nchunks, X, LB, values, meta, scale, T, stream);
            break;
        case 3:
            launch_rt<3>(rowt, M, K, nchunks, X, LB, values, meta, scale, T, stream);
            break;
        default:
            launch_rt<4>(rowt, M, K, nchunks, X, LB, values, meta, scale, T, stream);
            break;
    }
    return launch_status();
}

}  // namespace lynx
