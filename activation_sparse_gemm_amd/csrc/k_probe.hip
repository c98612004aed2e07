// Test hooks: one matrix instruction per wave on raw per-lane register
// contents (declared in lynx_probe.h).  Each kernel is launched as exactly one
// workgroup of 64 lanes; lane l reads and writes only its own slots.
#include "lynx_internal.h"
#include "lynx_probe.h"

namespace lynx {
namespace {

template <int ABID>
__global__ __launch_bounds__(64) void probe_smfmac_16x16x64(const bf16x8* a, const bf16x16* b,
                                                            const uint32_t* idx, f32x4* d) {
    const int l = threadIdx.x;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a[l], b[l], acc, (int)idx[l], 0, ABID);
    d[l] = acc;
}

template <int ABID>
__global__ __launch_bounds__(64) void probe_smfmac_32x32x32(const bf16x8* a, const bf16x16* b,
                                                            const uint32_t* idx, f32x16* d) {
    const int l = threadIdx.x;
    f32x16 acc = {};
    acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[l], b[l], acc, (int)idx[l], 0, ABID);
    d[l] = acc;
}

__global__ __launch_bounds__(64) void probe_mfma_16x16x32(const bf16x8* a, const bf16x8* b,
                                                          f32x4* d) {
    const int l = threadIdx.x;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[l], b[l], acc, 0, 0, 0);
    d[l] = acc;
}

__global__ __launch_bounds__(64) void probe_mfma_32x32x16(const bf16x8* a, const bf16x8* b,
                                                          f32x16* d) {
    const int l = threadIdx.x;
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[l], b[l], acc, 0, 0, 0);
    d[l] = acc;
}

}  // namespace
}  // namespace lynx

using namespace lynx;

extern "C" lynx_status lynx_probe_mfma(int which, int abid, const uint16_t* a, const uint16_t* b,
                                       const uint32_t* idx, float* d, lynx_stream_t stream) {
    if (which < 0 || which > 3 || abid < 0 || abid > 1) return LYNX_ERR_SHAPE;
    if (!a || !b || !d || (which < 2 && !idx)) return LYNX_ERR_NULL;
    if (!aligned16(a) || !aligned16(b) || !aligned16(d) || (which < 2 && !aligned16(idx)))
        return LYNX_ERR_ALIGN;
    lynx_status st = check_device();
    if (st != LYNX_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bf16x8* A = reinterpret_cast<const bf16x8*>(a);
    switch (which) {
        case 0: {
            const bf16x16* B = reinterpret_cast<const bf16x16*>(b);
            f32x4* D = reinterpret_cast<f32x4*>(d);
            if (abid == 0)
                hipLaunchKernelGGL(probe_smfmac_16x16x64<0>, dim3(1), dim3(64), 0, s, A, B, idx, D);
            else
                hipLaunchKernelGGL(probe_smfmac_16x16x64<1>, dim3(1), dim3(64), 0, s, A, B, idx, D);
            break;
        }
        case 1: {
            const bf16x16* B = reinterpret_cast<const bf16x16*>(b);
            f32x16* D = reinterpret_cast<f32x16*>(d);
            if (abid == 0)
                hipLaunchKernelGGL(probe_smfmac_32x32x32<0>, dim3(1), dim3(64), 0, s, A, B, idx, D);
            else
                hipLaunchKernelGGL(probe_smfmac_32x32x32<1>, dim3(1), dim3(64), 0, s, A, B, idx, D);
            break;
        }
        case 2:
            hipLaunchKernelGGL(probe_mfma_16x16x32, dim3(1), dim3(64), 0, s, A,
                               reinterpret_cast<const bf16x8*>(b), reinterpret_cast<f32x4*>(d));
            break;
        default:
            hipLaunchKernelGGL(probe_mfma_32x32x16, dim3(1), dim3(64), 0, s, A,
                               reinterpret_cast<const bf16x8*>(b), reinterpret_cast<f32x16*>(d));
            break;
    }
    return launch_status();
}
