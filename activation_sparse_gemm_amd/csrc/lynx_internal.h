// Internal declarations shared by the liblynx translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lynx.h"

namespace lynx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Checks that the current device is gfx950 (cached per device ordinal).
lynx_status check_device();

// Number of compute units of the current device (cached per device ordinal).
lynx_status device_cu_count(int* cus);

// Maps the last HIP launch error to a status.
inline lynx_status launch_status() {
    return hipGetLastError() == hipSuccess ? LYNX_OK : LYNX_ERR_DEVICE;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- the sparse layer, shared by the entry points -------------------------
// Argument checks of the sparse + LoRA layer (everything but its workspace);
// LYNX_OK with *noop set when M or N is 0.
lynx_status validate_sparse_layer(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                                  const uint16_t* LB, const uint16_t* Y, int64_t M, int64_t N,
                                  int64_t K, int64_t R, bool* noop);

// Workspace bytes of the sparse layer (valid sizes only; 0 if the device
// cannot be queried).
size_t sparse_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t R);

// The sparsifier then the sparse GEMM, on validated arguments, with the
// packed operand, s, T and the GEMM's stream-K partial sums in `workspace`
// (sparse_workspace_bytes, 256-byte aligned).
lynx_status run_sparse_layer(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                             const uint16_t* LB, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                             int64_t R, void* workspace, hipStream_t s);

// ---- schedule of the sparse GEMM (k_dispatch.hip) --------------------------
// Tiled kernel or 64 x 64 kernel; for the tiled kernel the tile width and
// the split of the tiles into whole tiles and stream-K tiles (whose 64-channel
// stages are spread evenly over the workgroups, partial sums handed over in
// the workspace).
struct SparsePlan {
    bool tiled;            // tiled kernel (k_gemm.hip), else the 64 x 64 kernel
    int nb;                // tile width 64 * nb: 4 (256) or 3 (192)
    int grid;              // persistent workgroups
    int dp_tiles;          // whole tiles
    int sk_tiles;          // stream-K tiles (0: none)
    int pairs;             // 64-channel stage pairs of the stream-K tiles
    size_t partial_bytes;  // one slot of fp32 accumulators per workgroup (0: no stream-K)
    size_t flag_bytes;     // one int per stream-K tile, 256-byte rounded (0: no stream-K)
};
// with_sk: stream-K allowed (the caller has a workspace for it).  Depends on
// the current device's compute-unit count; where no device can be queried
// (a host without a GPU) it assumes the MI355X's 256.
SparsePlan plan_sparse_gemm(int M, int N, int K, bool with_sk);
// the same for a device of `cus` compute units
SparsePlan plan_sparse_gemm_for(int M, int N, int K, bool with_sk, int cus);

// ---- kernel launchers (validated arguments only) ---------------------------
// zero_flags / nzero: ints the sparsifier clears (the GEMM's stream-K flags)
lynx_status launch_sparsify(const uint16_t* X, const uint16_t* LB, int M, int K, int R,
                            uint16_t* values, uint8_t* meta, float* scale, uint16_t* T,
                            int* zero_flags, int nzero, hipStream_t stream);

// sets n ints to zero (a kernel, so it may be captured in a graph)
lynx_status launch_zero_ints(int* p, int n, hipStream_t stream);

// partials / flags: the plan's stream-K workspace (flags zero), unused without
lynx_status launch_gemm_sparse(const uint16_t* values, const uint8_t* meta, const float* scale,
                               const uint16_t* T, const uint16_t* W, const uint16_t* LA,
                               uint16_t* Y, int M, int N, int K, int R, const SparsePlan& plan,
                               float* partials, int* flags, hipStream_t stream);

lynx_status launch_gemm_dense(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N,
                              int K, hipStream_t stream);

}  // namespace lynx
