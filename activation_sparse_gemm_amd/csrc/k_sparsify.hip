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
//   workgroup = 16 rows (tokens) x all of K; waves split K in 128-channel chunks.
//   lane l: row r = l % 16, quarter q = l / 16; in chunk c it owns channels
//   [128c + 32q, 128c + 32q + 32): 8 groups of 4, loaded as 4 x 16 bytes.
//   - selection + packing in registers: 16 kept values (32 B) and 8 codes (4 B)
//     per lane and chunk, stored in the 16-row x 64-channel tile order of the
//     packed operand (a workgroup's 16 rows are exactly one tile row-block;
//     rows past M are written as zero values and codes (0,1));
//   - row norms ||x||^2 and ||x~||^2 with v_dot2_f32_bf16 (products of bf16 are
//     exact in fp32), summed per chunk in fp32 then in fp64;
//   - T: the lane's 32 channels are the A operand of 4 v_mfma_f32_16x16x32_bf16
//     steps (k-block q of each step), LB rows supply the B operand with the same
//     channel map, one 16-column tile of T per 16 ranks.
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
constexpr int kMaxWaves = 8;

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

template <int RT>  // RT = R / 16 column tiles of T (0..4)
__global__ __launch_bounds__(kMaxWaves * 64) void sparsify_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ LB, int M, int K,
    uint16_t* __restrict__ values, uint8_t* __restrict__ meta, float* __restrict__ scale,
    uint16_t* __restrict__ T) {
    constexpr int R = RT * 16;
    __shared__ double red_norm[kMaxWaves][kRows][2];
    __shared__ int exact_row[kRows];
    // per-wave LB chunk (R rows x 256 B, XOR-swizzled 16-byte pieces); after
    // the main loop the same memory holds the cross-wave T partials
    constexpr int kLbBytes = RT > 0 ? R * 256 : 64;
    __shared__ __attribute__((aligned(16))) char lbw[kMaxWaves][kLbBytes];
    static_assert(sizeof(lbw) >= sizeof(float) * kMaxWaves * kRows * (RT > 0 ? R : 1),
                  "T partials fit in the LB staging area");
    float(*red_T)[kRows][RT > 0 ? R : 1] =
        reinterpret_cast<float(*)[kRows][RT > 0 ? R : 1]>(&lbw[0][0]);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int r = lane & 15;
    const int q = lane >> 4;
    const int m0 = blockIdx.x * kRows;
    const int row = m0 + r;
    const bool row_ok = row < M;
    const int nchunks = K / kChunk;

    const uint16_t* xrow = X + size_t(row_ok ? row : M - 1) * size_t(K);
    // packed operand, tile order: tile (block b, 64-channel step s) holds 16 rows
    // x 32 values (1 KB) and 16 rows x 8 meta bytes (128 B)
    const int steps = K / 64;
    uint16_t* vtile = values + size_t(blockIdx.x) * size_t(steps) * 512 + r * 32;
    uint8_t* mtile = meta + size_t(blockIdx.x) * size_t(steps) * 128 + r * 8;

    f32x4 acc[RT > 0 ? RT : 1];
#pragma unroll
    for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    double n2 = 0.0, nt2 = 0.0;

    // X: the lane's 32 channels of a chunk.  LB: its rows x the chunk's 128
    // channels, read as whole row segments (instruction j: rows 4j .. 4j+3,
    // lane l -> row 4j + l / 16, 16-byte piece l % 16), later put in the
    // wave's LDS area for the MFMA B operand.  A wave walks its chunks one
    // after another, so each load is issued a chunk ahead: the next chunk's X
    // before this chunk is worked on, its LB as soon as this chunk's LB has
    // gone to the LDS (the same registers).
    auto load_x = [&](int c, u32x4* xd) {
        const int k = c * kChunk + q * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) xd[i] = *reinterpret_cast<const u32x4*>(xrow + k + 8 * i);
    };
    auto load_lb = [&](int c, u32x4* ld) {
#pragma unroll
        for (int j = 0; j < (RT > 0 ? R / 4 : 0); ++j) {
            const int lr = 4 * j + (lane >> 4);
            ld[j] = *reinterpret_cast<const u32x4*>(LB + size_t(lr) * size_t(K) +
                                                    size_t(c) * kChunk + 8 * (lane & 15));
        }
    };
    u32x4 xv[4], lbraw[RT > 0 ? R / 4 : 1];
    if (wave < nchunks) {
        load_x(wave, xv);
        load_lb(wave, lbraw);
    }

    for (int c = wave; c < nchunks; c += nwaves) {
        const int k = c * kChunk + q * 32;
        const bool more = c + nwaves < nchunks;
        u32x4 xn[4];
        if (more) load_x(c + nwaves, xn);

        // dense row norm
        float pn = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pn = dot2_self(xv[i].x, pn);
            pn = dot2_self(xv[i].y, pn);
            pn = dot2_self(xv[i].z, pn);
            pn = dot2_self(xv[i].w, pn);
        }

        // selection and packing: group g of this lane is dwords 2g, 2g+1
        uint32_t kept[8];
        uint32_t code = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            code |= select_group(xv[i].x, xv[i].y, kept[2 * i]) << (8 * i);
            code |= select_group(xv[i].z, xv[i].w, kept[2 * i + 1]) << (8 * i + 4);
        }
        float pt = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) pt = dot2_self(kept[g], pt);
        n2 += double(pn);
        nt2 += double(pt);

        {
            // channels k .. k+31 = half (q & 1) of step k / 64
            const int step = k >> 6, half = q & 1;
            u32x4* vdst = reinterpret_cast<u32x4*>(vtile + step * 512 + half * 16);
            uint32_t* mdst = reinterpret_cast<uint32_t*>(mtile + step * 128 + half * 4);
            if (row_ok) {
                vdst[0] = u32x4{kept[0], kept[1], kept[2], kept[3]};
                vdst[1] = u32x4{kept[4], kept[5], kept[6], kept[7]};
                *mdst = code;
            } else {
                vdst[0] = u32x4{0u, 0u, 0u, 0u};
                vdst[1] = u32x4{0u, 0u, 0u, 0u};
                *mdst = 0x44444444u;
            }
        }

        // T += X LB^T over these channels; B operand of step i: LB row
        // 16 t + r, channels 32 q + 8 i .. +8 of the chunk
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
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, xv[i]), bv, acc[t], 0, 0, 0);
                }
            }
            // the next chunk's writes must not overtake this chunk's reads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[i] = xn[i];
        }
    }

    // ---- cross-lane (4 quarters of a row) then cross-wave reductions ----
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    nt2 += __shfl_xor(nt2, 16);
    nt2 += __shfl_xor(nt2, 32);
    if (q == 0) {
        red_norm[wave][r][0] = n2;
        red_norm[wave][r][1] = nt2;
    }
    __syncthreads();  // every wave is done with its LB area before it holds T partials
    // accumulator layout of a 16x16 tile: lane (n = l % 16, q) holds rows 4q..4q+3
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red_T[wave][4 * q + e][16 * t + r] = acc[t][e];
    }
    __syncthreads();

    if (threadIdx.x < kRows) {
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
    __syncthreads();
    // exact fp64 pass for rows outside the fast path's range (rare)
    for (int rr = wave; rr < kRows; rr += nwaves) {
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
    if constexpr (RT > 0) {
        for (int idx = threadIdx.x; idx < kRows * R; idx += blockDim.x) {
            const int rr = idx / R, cc = idx % R;
            float s = 0.f;
            for (int w = 0; w < nwaves; ++w) s += red_T[w][rr][cc];
            if (m0 + rr < M)
                T[size_t(m0 + rr) * R + cc] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(s));
        }
    }
}

}  // namespace

lynx_status launch_sparsify(const uint16_t* X, const uint16_t* LB, int M, int K, int R,
                            uint16_t* values, uint8_t* meta, float* scale, uint16_t* T,
                            hipStream_t stream) {
    const int nchunks = K / kChunk;
    const int nwaves = nchunks < kMaxWaves ? nchunks : kMaxWaves;
    const dim3 grid((M + kRows - 1) / kRows), block(64 * nwaves);
    switch (R / 16) {
        case 0:
            hipLaunchKernelGGL(sparsify_kernel<0>, grid, block, 0, stream, X, LB, M, K, values,
                               meta, scale, T);
            break;
        case 1:
            hipLaunchKernelGGL(sparsify_kernel<1>, grid, block, 0, stream, X, LB, M, K, values,
                               meta, scale, T);
            break;
        case 2:
            hipLaunchKernelGGL(sparsify_kernel<2>, grid, block, 0, stream, X, LB, M, K, values,
                               meta, scale, T);
            break;
        case 3:
            hipLaunchKernelGGL(sparsify_kernel<3>, grid, block, 0, stream, X, LB, M, K, values,
                               meta, scale, T);
            break;
        default:
            hipLaunchKernelGGL(sparsify_kernel<4>, grid, block, 0, stream, X, LB, M, K, values,
                               meta, scale, T);
            break;
    }
    return launch_status();
}

}  // namespace lynx
