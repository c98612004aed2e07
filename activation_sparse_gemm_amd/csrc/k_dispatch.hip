// Kernel selection for the GEMM entry points.  Problems that give at least 16
// output tiles of 256 x 256 and have K >= 128 run the tiled kernels
// (k_gemm.hip, k_gemm_dense.hip: their LDS rings need two 64-channel stages);
// smaller ones, which cannot fill the chip with 256 x 256 tiles and are
// launch-bound, and K = 64, run the 64 x 64 kernels (k_gemm_ref.hip).
#include "lynx_internal.h"

namespace lynx {

lynx_status launch_gemm_sparse_ref(const uint16_t* values, const uint8_t* meta,
                                   const float* scale, const uint16_t* T, const uint16_t* W,
                                   const uint16_t* LA, uint16_t* Y, int M, int N, int K, int R,
                                   hipStream_t stream);
lynx_status launch_gemm_dense_ref(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N,
                                  int K, hipStream_t stream);
lynx_status launch_gemm_sparse_tiled(const uint16_t* values, const uint8_t* meta,
                                     const float* scale, const uint16_t* T, const uint16_t* W,
                                     const uint16_t* LA, uint16_t* Y, int M, int N, int K, int R,
                                     hipStream_t stream);
lynx_status launch_gemm_dense_tiled(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M,
                                    int N, int K, hipStream_t stream);

namespace {
bool use_tiled(int M, int N, int K) {
    const long tiles = long((M + 255) / 256) * long((N + 255) / 256);
    return tiles >= 16 && K >= 128;
}
}  // namespace

lynx_status launch_gemm_sparse(const uint16_t* values, const uint8_t* meta, const float* scale,
                               const uint16_t* T, const uint16_t* W, const uint16_t* LA,
                               uint16_t* Y, int M, int N, int K, int R, hipStream_t stream) {
    if (use_tiled(M, N, K))
        return launch_gemm_sparse_tiled(values, meta, scale, T, W, LA, Y, M, N, K, R, stream);
    return launch_gemm_sparse_ref(values, meta, scale, T, W, LA, Y, M, N, K, R, stream);
}

lynx_status launch_gemm_dense(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N,
                              int K, hipStream_t stream) {
    if (use_tiled(M, N, K)) return launch_gemm_dense_tiled(X, W, Y, M, N, K, stream);
    return launch_gemm_dense_ref(X, W, Y, M, N, K, stream);
}

}  // namespace lynx
