// Test hooks: one matrix instruction per wave on raw per-lane register
// contents (declared in lynx_probe.h).  Each kernel is launched as exactly one
// workgroup of 64 lanes; lane l reads and writes only its own slots.
#include <type_traits>

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

// Issue-rate probe: every wave runs `iters` rounds of 16 matrix instructions
// over 4 independent accumulators (so no instruction waits for the previous
// one's result), between two stamps of the shader-clock counter (s_memtime)
// and the 100 MHz real-time counter (s_memrealtime).  Operands are formed
// from the lane id; the accumulators are summed into `sink` so nothing is
// removed by the compiler.
template <int WHICH>
__global__ __launch_bounds__(256) void probe_rate(int iters, float* sink, uint64_t* stamps) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const float fl = 1.0f + 0x1p-8f * float(lane & 7);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(fl);
        b[i] = static_cast<__bf16>(0x1p-12f * float(i + 1));
    }
    const bf16x16 b16 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 3, 4, 5, 6, 7);
    const int idx = 0x4444;  // positions 0 and 1 of every group
    constexpr bool kSmall = WHICH == 0 || WHICH == 2;
    typedef typename std::conditional<kSmall, f32x4, f32x16>::type acc_t;
    acc_t acc[4] = {};
    __builtin_amdgcn_s_waitcnt(0);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if constexpr (WHICH == 0)
                acc[j & 3] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b16, acc[j & 3], idx, 0, 0);
            else if constexpr (WHICH == 1)
                acc[j & 3] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b16, acc[j & 3], idx, 0, 0);
            else if constexpr (WHICH == 2)
                acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j & 3], 0, 0, 0);
            else
                acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j & 3], 0, 0, 0);
        }
    }
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < int(sizeof(acc_t) / 4); ++e) v += acc[j][e];
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    sink[blockIdx.x * 256 + threadIdx.x] = v;
    if (lane == 0) {
        uint64_t* st = stamps + (size_t(blockIdx.x) * 4 + wave) * 2;
        st[0] = t1 - t0;
        st[1] = r1 - r0;
    }
}

}  // namespace
}  // namespace lynx

using namespace lynx;

extern "C" lynx_status lynx_probe_mfma_rate(int which, int iters, int grid, float* sink,
                                            uint64_t* stamps, lynx_stream_t stream) {
    if (which < 0 || which > 3 || iters < 1 || grid < 1) return LYNX_ERR_SHAPE;
    if (!sink || !stamps) return LYNX_ERR_NULL;
    if (!aligned16(sink) || !aligned16(stamps)) return LYNX_ERR_ALIGN;
    lynx_status st = check_device();
    if (st != LYNX_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (which) {
        case 0: hipLaunchKernelGGL(probe_rate<0>, dim3(grid), dim3(256), 0, s, iters, sink, stamps); break;
        case 1: hipLaunchKernelGGL(probe_rate<1>, dim3(grid), dim3(256), 0, s, iters, sink, stamps); break;
        case 2: hipLaunchKernelGGL(probe_rate<2>, dim3(grid), dim3(256), 0, s, iters, sink, stamps); break;
        default: hipLaunchKernelGGL(probe_rate<3>, dim3(grid), dim3(256), 0, s, iters, sink, stamps); break;
    }
    return launch_status();
}

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
