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

// Workspace bytes of the sparse layer (valid sizes only).
size_t sparse_workspace_bytes(int64_t M, int64_t K, int64_t R);

// The sparsifier then the sparse GEMM, on validated arguments, with the
// packed operand, s and T in `workspace` (sparse_workspace_bytes, 256-byte
// aligned).
lynx_status run_sparse_layer(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                             const uint16_t* LB, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                             int64_t R, void* workspace, hipStream_t s);

// ---- kernel launchers (validated arguments only) ---------------------------
lynx_status launch_sparsify(const uint16_t* X, const uint16_t* LB, int M, int K, int R,
                            uint16_t* values, uint8_t* meta, float* scale, uint16_t* T,
                            hipStream_t stream);

lynx_status launch_gemm_sparse(const uint16_t* values, const uint8_t* meta, const float* scale,
                               const uint16_t* T, const uint16_t* W, const uint16_t* LA,
                               uint16_t* Y, int M, int N, int K, int R, hipStream_t stream);

lynx_status launch_gemm_dense(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N,
                              int K, hipStream_t stream);

}  // namespace lynx
