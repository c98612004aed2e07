// Straightforward GEMM kernels: operands read from global memory straight
// into the matrix-instruction register layouts, one 64x64 output tile per
// workgroup.  They are the simplest correct form of K2 (2:4 sparse MFMA with
// the LoRA epilogue) and K3 (dense MFMA), used for shapes the tiled kernels
// do not take and as a second device implementation in the tests.
//
// Layer (RT-Lynx page, 코드 예제, second formula; 방법론 "CUDA 커널 최적화":
// the LoRA output is accumulated on chip inside the sparse GEMM):
//   Y = s * (X~ W^T) + T LA^T,  T = X LB^T.
//
// Register layouts (gfx950, pinned by the probe tests), lane l, r = l % 16,
// q = l / 16:
//   v_smfmac_f32_16x16x64_bf16 (64-channel step): A = row r, dense channels
//     [16q, 16q + 16) as 8 kept values + a 16-bit index word (group g of the
//     lane in bits 4g..4g+3, first kept position in the low 2 bits);
//     B = column r, elements 0..7 = channels [8q, 8q + 8), elements 8..15 =
//     channels [32 + 8q, 40 + 8q).
//   v_mfma_f32_16x16x32_bf16: A = row r, channels [8q, 8q + 8); B = column r,
//     channels [8q, 8q + 8).
//   16x16 accumulator: column r, rows 4q .. 4q + 3.
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kTile = 64;

__device__ __forceinline__ void store_tile_bf16(uint16_t* Y, int M, int N, int row0, int col,
                                                const f32x4& v) {
    if (col >= N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = row0 + e;
        if (row < M)
            Y[size_t(row) * size_t(N) + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[e]));
    }
}

// LoRA up-projection of a 32x32 sub-tile: acc2[a][b] += T[rows a] LA[cols b]^T.
__device__ __forceinline__ void lora_up(const uint16_t* T, const uint16_t* LA, int R,
                                        const int am[2], const int bn[2], int q,
                                        f32x4 acc2[2][2]) {
    for (int kr = 0; kr < R; kr += 32) {
        const int kc = kr + 8 * q;
        const bool live = kc < R;  // R % 32 == 16: upper half of the last step is zero
        bf16x8 ta[2], lb[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            ta[a] = live ? *reinterpret_cast<const bf16x8*>(T + size_t(am[a]) * R + kc) : bf16x8{};
#pragma unroll
        for (int b = 0; b < 2; ++b)
            lb[b] = live ? *reinterpret_cast<const bf16x8*>(LA + size_t(bn[b]) * R + kc) : bf16x8{};
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc2[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta[a], lb[b], acc2[a][b], 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void gemm_sparse_ref(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta,
    const float* __restrict__ scale, const uint16_t* __restrict__ T, const uint16_t* __restrict__ W,
    const uint16_t* __restrict__ LA, uint16_t* __restrict__ Y, int M, int N, int K, int R) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = blockIdx.y * kTile + 32 * wm, n0 = blockIdx.x * kTile + 32 * wn;
    int am[2], bn[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        am[i] = min(m0 + 16 * i + r, M - 1);  // clamped rows/cols are computed, never stored
        bn[i] = min(n0 + 16 * i + r, N - 1);
    }
    f32x4 acc[2][2] = {}, acc2[2][2] = {};
    for (int kk = 0; kk < K; kk += 64) {
        bf16x8 A[2];
        uint32_t I[2];
        bf16x16 B[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            // packed operand in 16-row x 64-channel tiles (512 values, 128 meta bytes)
            const size_t tile = size_t(am[a] >> 4) * size_t(K / 64) + size_t(kk / 64);
            const int rr = am[a] & 15;
            A[a] = *reinterpret_cast<const bf16x8*>(values + tile * 512 + rr * 32 + 8 * q);
            I[a] = *reinterpret_cast<const uint16_t*>(meta + tile * 128 + rr * 8 + 2 * q);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint16_t* wrow = W + size_t(bn[b]) * K + kk + 8 * q;
            const bf16x8 lo = *reinterpret_cast<const bf16x8*>(wrow);
            const bf16x8 hi = *reinterpret_cast<const bf16x8*>(wrow + 32);
            B[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[a][b] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(A[a], B[b], acc[a][b],
                                                                      (int)I[a], 0, 0);
    }
    if (R > 0) lora_up(T, LA, R, am, bn, q, acc2);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int row0 = m0 + 16 * a + 4 * q;
        f32x4 s;
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = scale[min(row0 + e, M - 1)];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = s[e] * acc[a][b][e] + acc2[a][b][e];
            store_tile_bf16(Y, M, N, row0, n0 + 16 * b + r, y);
        }
    }
}

__global__ __launch_bounds__(256) void gemm_dense_ref(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W,
                                                      uint16_t* __restrict__ Y, int M, int N,
                                                      int K) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = blockIdx.y * kTile + 32 * wm, n0 = blockIdx.x * kTile + 32 * wn;
    int am[2], bn[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        am[i] = min(m0 + 16 * i + r, M - 1);
        bn[i] = min(n0 + 16 * i + r, N - 1);
    }
    f32x4 acc[2][2] = {};
    for (int kk = 0; kk < K; kk += 32) {
        bf16x8 A[2], B[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            A[a] = *reinterpret_cast<const bf16x8*>(X + size_t(am[a]) * K + kk + 8 * q);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            B[b] = *reinterpret_cast<const bf16x8*>(W + size_t(bn[b]) * K + kk + 8 * q);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[a], B[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            store_tile_bf16(Y, M, N, m0 + 16 * a + 4 * q, n0 + 16 * b + r, acc[a][b]);
}

}  // namespace

lynx_status launch_gemm_sparse_ref(const uint16_t* values, const uint8_t* meta,
                                   const float* scale, const uint16_t* T, const uint16_t* W,
                                   const uint16_t* LA, uint16_t* Y, int M, int N, int K, int R,
                                   hipStream_t stream) {
    const dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile), block(256);
    hipLaunchKernelGGL(gemm_sparse_ref, grid, block, 0, stream, values, meta, scale, T, W, LA, Y,
                       M, N, K, R);
    return launch_status();
}

lynx_status launch_gemm_dense_ref(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N,
                                  int K, hipStream_t stream) {
    const dim3 grid((N + kTile - 1) / kTile, (M + kTile - 1) / kTile), block(256);
    hipLaunchKernelGGL(gemm_dense_ref, grid, block, 0, stream, X, W, Y, M, N, K);
    return launch_status();
}

}  // namespace lynx
