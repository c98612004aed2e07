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
// 128 x 128 = 8 x 8 accumulator tiles of 16 x 16 (256 fp32 per lane).  The K
// loop moves 64 dense channels per stage through LDS, double-buffered; global
// loads for stage t+1 are in flight while stage t is multiplied.
//   sparse stage: A = packed values 256 rows x 64 B, meta 256 rows x 8 B,
//                 B = W 256 rows x 128 B               (50 KB)
//   dense stage:  A = X 256 rows x 128 B, B = W 256 rows x 128 B   (64 KB)
// LDS rows are stored with their 16-byte chunks XOR-swizzled by row so that
// the 16-byte fragment reads of 8 (or 16) consecutive lanes hit distinct banks.
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

constexpr int BM = 256, BN = 256, BK = 64, NT = 256, GROUP_M = 8;

template <bool SPARSE>
struct Cfg {
    static constexpr int A_ROW = SPARSE ? 64 : 128;  // bytes per A row per stage
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int META_BYTES = SPARSE ? BM * 8 : 0;
    static constexpr int B_BYTES = BN * 128;
    static constexpr int STAGE = A_BYTES + META_BYTES + B_BYTES;
    static constexpr int A_LOADS = A_BYTES / 16 / NT;  // 16-byte chunks per thread
    static constexpr int B_LOADS = B_BYTES / 16 / NT;
    static constexpr int EPI_OFF = 64 * 1024;             // epilogue scratch, 4 KB per wave
    static constexpr int LDS = (2 * STAGE > EPI_OFF + 4 * 4096) ? 2 * STAGE : EPI_OFF + 4 * 4096;
};

// chunk swizzles (16-byte chunk index within a row)
__device__ __forceinline__ int swz128(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

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
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- staging: buffer loads (rows past M or N read as zero) -------------
    // Thread tid moves chunk c = tid + 256 j (j = 0..) of each operand per stage.
    // Consecutive j are a fixed number of rows apart, so one per-thread byte
    // offset plus a uniform per-j offset addresses every chunk, and the LDS
    // swizzle (a function of row % 16) is the same for every j.
    const int rowbytesA = SPARSE ? K : 2 * K;  // packed values: K/2 bf16 per row
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Aptr), (short)0, M * rowbytesA, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(W), (short)0, N * 2 * K, 0x00020000);
    constexpr int A_ROWS_PER_J = SPARSE ? 64 : 32;  // NT chunks cover this many rows
    int voffA, dstA0;
    if constexpr (SPARSE) {
        const int row = tid >> 2, ch = tid & 3;
        voffA = (m0 + row) * rowbytesA + ch * 16;
        dstA0 = row * 64 + 16 * (ch ^ swz64(row));
    } else {
        const int row = tid >> 3, ch = tid & 7;
        voffA = (m0 + row) * rowbytesA + ch * 16;
        dstA0 = row * 128 + 16 * (ch ^ swz128(row));
    }
    const int voffB = (n0 + (tid >> 3)) * 2 * K + (tid & 7) * 16;
    const int dstB0 = C::A_BYTES + C::META_BYTES + (tid >> 3) * 128 +
                      16 * ((tid & 7) ^ swz128(tid >> 3));
    __amdgpu_buffer_rsrc_t rsM;
    int voffM = 0;
    if constexpr (SPARSE) {
        rsM = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(meta), (short)0, M * (K / 8),
                                                0x00020000);
        voffM = (m0 + tid) * (K / 8);
    }

    u32x4 stA[C::A_LOADS], stB[C::B_LOADS];
    u32x2 stM = {0u, 0u};

    auto load_global = [&](int kk) {
        const int kbA = SPARSE ? kk : 2 * kk;  // byte offset of this stage in an A row
#pragma unroll
        for (int j = 0; j < C::A_LOADS; ++j)
            stA[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rsA, voffA, j * A_ROWS_PER_J * rowbytesA + kbA, 0));
#pragma unroll
        for (int j = 0; j < C::B_LOADS; ++j)
            stB[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rsB, voffB, j * 32 * 2 * K + 2 * kk, 0));
        if constexpr (SPARSE)
            stM = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsM, voffM, kk / 8, 0));
    };
    auto store_lds = [&](char* buf) {
#pragma unroll
        for (int j = 0; j < C::A_LOADS; ++j) *reinterpret_cast<u32x4*>(buf + dstA0 + 4096 * j) = stA[j];
#pragma unroll
        for (int j = 0; j < C::B_LOADS; ++j) *reinterpret_cast<u32x4*>(buf + dstB0 + 4096 * j) = stB[j];
        if constexpr (SPARSE) *reinterpret_cast<u32x2*>(buf + C::A_BYTES + tid * 8) = stM;
    };

    // ---- per-lane fragment offsets (swizzle depends on row % 16 = r only) --
    const int sw128 = swz128(r), sw64 = swz64(r);
    const int rowA = wm * 128 + r, rowB = wn * 128 + r;

    f32x4 acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    load_global(0);
    store_lds(smem);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        char* cur = smem + (t & 1) * C::STAGE;
        char* nxt = smem + ((t + 1) & 1) * C::STAGE;
        if (t + 1 < nk) load_global((t + 1) * BK);

        if constexpr (SPARSE) {
            const char* As = cur;
            const char* Ms = cur + C::A_BYTES;
            const char* Bs = cur + C::A_BYTES + C::META_BYTES;
            bf16x16 bfr[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int base = (rowB + 16 * b) * 128;
                const bf16x8 lo = lds_read<bf16x8>(Bs, base + 16 * (q ^ sw128));
                const bf16x8 hi = lds_read<bf16x8>(Bs, base + 16 * ((4 + q) ^ sw128));
                bfr[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                                 12, 13, 14, 15);
            }
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const int row = rowA + 16 * a;
                const bf16x8 afr = lds_read<bf16x8>(As, row * 64 + 16 * (q ^ sw64));
                const int idx = lds_read<uint16_t>(Ms, row * 8 + 2 * q);
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    acc[a][b] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(afr, bfr[b], acc[a][b],
                                                                          idx, 0, 0);
            }
        } else {
            const char* As = cur;
            const char* Bs = cur + C::A_BYTES;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 bfr[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    bfr[b] = lds_read<bf16x8>(Bs, (rowB + 16 * b) * 128 + 16 * ((4 * ks + q) ^ sw128));
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    const bf16x8 afr =
                        lds_read<bf16x8>(As, (rowA + 16 * a) * 128 + 16 * ((4 * ks + q) ^ sw128));
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[b], acc[a][b],
                                                                            0, 0, 0);
                }
            }
        }

        if (t + 1 < nk) store_lds(nxt);
        __syncthreads();
    }

    // ---- LoRA up-projection: acc += (T / s) LA^T  ----------------------------
    if constexpr (SPARSE) {
        if (R > 0) {
            // stage T / s (rows m0..) and LA (rows n0..), 256 x 64 bf16 each,
            // zero beyond R, same swizzled 128-byte rows as the dense tiles
            char* Ts = smem;
            char* Ls = smem + 32 * 1024;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = tid + NT * j;
                const int row = c >> 3, ch = c & 7;
                const int off = row * 128 + 16 * (ch ^ swz128(row));
                u32x4 tv = {0u, 0u, 0u, 0u}, lv = {0u, 0u, 0u, 0u};
                if (ch * 8 < R) {
                    const int gm = min(m0 + row, M - 1);
                    const u32x4 raw = *reinterpret_cast<const u32x4*>(T + size_t(gm) * R + ch * 8);
                    const float inv = 1.0f / scale[gm];
                    tv.x = pack_bf16x2(bf16_lo(raw.x) * inv, bf16_hi(raw.x) * inv);
                    tv.y = pack_bf16x2(bf16_lo(raw.y) * inv, bf16_hi(raw.y) * inv);
                    tv.z = pack_bf16x2(bf16_lo(raw.z) * inv, bf16_hi(raw.z) * inv);
                    tv.w = pack_bf16x2(bf16_lo(raw.w) * inv, bf16_hi(raw.w) * inv);
                    lv = *reinterpret_cast<const u32x4*>(LA + size_t(min(n0 + row, N - 1)) * R +
                                                          ch * 8);
                }
                *reinterpret_cast<u32x4*>(Ts + off) = tv;
                *reinterpret_cast<u32x4*>(Ls + off) = lv;
            }
            __syncthreads();
            for (int ks = 0; ks < (R + 31) / 32; ++ks) {
                bf16x8 bfr[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    bfr[b] = lds_read<bf16x8>(Ls, (rowB + 16 * b) * 128 + 16 * ((4 * ks + q) ^ sw128));
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    const bf16x8 afr =
                        lds_read<bf16x8>(Ts, (rowA + 16 * a) * 128 + 16 * ((4 * ks + q) ^ sw128));
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
        float s4[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (SPARSE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] = scale[min(m0 + wm * 128 + row_l + e, M - 1)];
        }
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
