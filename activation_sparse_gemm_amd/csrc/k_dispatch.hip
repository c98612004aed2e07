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
                                     const SparsePlan& plan, float* partials, int* flags,
                                     hipStream_t stream);
lynx_status launch_gemm_dense_tiled(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M,
                                    int N, int K, hipStream_t stream);

namespace {
__global__ __launch_bounds__(256) void zero_ints(int* __restrict__ p, int n) {
    for (int i = int(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += int(gridDim.x * blockDim.x))
        p[i] = 0;
}

bool use_tiled(int M, int N, int K) {
    const long tiles = long((M + 255) / 256) * long((N + 255) / 256);
    return tiles >= 16 && K >= 128;
}

// Cost model of the tiled sparse GEMM, in shader cycles per workgroup,
// measured on the MI355X (per-wave cycle stamps at K = 3072, rank-64 LoRA):
// a 64-channel stage of a 256-wide tile takes 1414 cycles, of a 192-wide tile
// 1217; the LoRA step, scaling and stores of a tile 15.7 k and 11.7 k.  A
// stream-K range adds a segment start and the hand-over of one partial sum
// (about 6 k), and an owner reads one partial sum per other range in its
// tile (about 5 k each).
constexpr double kStageCycles[5] = {0, 0, 0, 1217.0, 1414.0};
constexpr double kTileEndCycles[5] = {0, 0, 0, 11700.0, 15700.0};
constexpr double kRangeCycles = 6000.0;
constexpr double kHandOverCycles = 5000.0;
// stream-K is taken only when the model puts it this much ahead
constexpr double kSkMargin = 0.02;

// Largest number of ranges that share one stream-K tile, with the kernel's
// split: range rho holds stage pairs floor(rho * pairs / P) ..
// floor((rho + 1) * pairs / P) - 1, and the range holding pair p is
// ceil((p + 1) * P / pairs) - 1.
int ranges_per_tile(long sk_tiles, long half_nk, int P) {
    const long pairs = sk_tiles * half_nk;
    auto range_of_pair = [&](long p) { return int(((p + 1) * P + pairs - 1) / pairs) - 1; };
    int most = 0;
    for (long t = 0; t < sk_tiles; ++t) {
        const int n = range_of_pair((t + 1) * half_nk - 1) - range_of_pair(t * half_nk) + 1;
        if (n > most) most = n;
    }
    return most;
}
}  // namespace

SparsePlan plan_sparse_gemm(int M, int N, int K, bool with_sk) {
    int cus = 0;
    if (device_cu_count(&cus) != LYNX_OK) cus = 256;
    return plan_sparse_gemm_for(M, N, K, with_sk, cus);
}

SparsePlan plan_sparse_gemm_for(int M, int N, int K, bool with_sk, int cus) {
    SparsePlan best{};
    best.tiled = use_tiled(M, N, K);
    if (!best.tiled) return best;
    const long nk = K / 64;
    const long tm = (M + 255) / 256;
    double best_cost = 0.0;
    for (int nb = 4; nb >= 3; --nb) {
        const long tiles = tm * ((N + 64 * nb - 1) / (64 * nb));
        const double tile = kStageCycles[nb] * double(nk) + kTileEndCycles[nb];
        // whole tiles only: rounds of tiles over the compute units
        const double whole = double((tiles + cus - 1) / cus) * tile;
        if (best_cost == 0.0 || whole < best_cost) {
            best_cost = whole;
            best.nb = nb;
            best.grid = int(tiles < cus ? tiles : cus);
            best.dp_tiles = int(tiles);
            best.sk_tiles = 0;
            best.pairs = 0;
        }
        if (!with_sk || nk % 2 != 0 || tiles % cus == 0) continue;
        // stream-K over the last partial round's tiles, or over those and one
        // full round more (ranges between one and two tiles long, which keeps
        // the tiles each range shares few)
        for (long extra = 0; extra <= 1; ++extra) {
            const long sk_tiles = tiles % cus + extra * cus;
            if (sk_tiles > tiles || sk_tiles * (nk / 2) < cus) continue;
            // the kernel's owners add at most two other ranges' partial sums
            if (ranges_per_tile(sk_tiles, nk / 2, cus) > 3) continue;
            const long dp_tiles = tiles - sk_tiles;
            const double c = double(dp_tiles / cus) * tile + double(sk_tiles) / cus * tile +
                             kRangeCycles + kHandOverCycles * double((cus + sk_tiles - 1) / sk_tiles);
            if (c * (1.0 + kSkMargin) < best_cost) {
                best_cost = c * (1.0 + kSkMargin);
                best.nb = nb;
                best.grid = cus;
                best.dp_tiles = int(dp_tiles);
                best.sk_tiles = int(sk_tiles);
                best.pairs = int(sk_tiles * (nk / 2));
            }
        }
    }
    if (best.sk_tiles > 0) {
        best.partial_bytes = size_t(best.grid) * size_t(4 * 64 * 64 * best.nb) * sizeof(float);
        best.flag_bytes = (size_t(best.sk_tiles) * sizeof(int) + 255) & ~size_t(255);
    }
    return best;
}

lynx_status launch_zero_ints(int* p, int n, hipStream_t stream) {
    if (n <= 0) return LYNX_OK;
    hipLaunchKernelGGL(zero_ints, dim3((n + 255) / 256 < 64 ? (n + 255) / 256 : 64), dim3(256), 0,
                       stream, p, n);
    return launch_status();
}

lynx_status launch_gemm_sparse(const uint16_t* values, const uint8_t* meta, const float* scale,
                               const uint16_t* T, const uint16_t* W, const uint16_t* LA,
                               uint16_t* Y, int M, int N, int K, int R, const SparsePlan& plan,
                               float* partials, int* flags, hipStream_t stream) {
    if (plan.tiled)
        return launch_gemm_sparse_tiled(values, meta, scale, T, W, LA, Y, M, N, K, R, plan,
                                        partials, flags, stream);
    return launch_gemm_sparse_ref(values, meta, scale, T, W, LA, Y, M, N, K, R, stream);
}

lynx_status launch_gemm_dense(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N,
                              int K, hipStream_t stream) {
    if (use_tiled(M, N, K)) return launch_gemm_dense_tiled(X, W, Y, M, N, K, stream);
    return launch_gemm_dense_ref(X, W, Y, M, N, K, stream);
}

}  // namespace lynx
