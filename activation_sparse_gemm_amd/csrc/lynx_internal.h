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
