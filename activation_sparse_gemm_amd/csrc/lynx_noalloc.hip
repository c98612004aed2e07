// lynx_linear_sparse_lora_noalloc: the sparse + LoRA layer with its workspace
// (packed operand, s, T) in a static device array, for callers that cannot
// allocate device memory (graph capture, serving loops, harnesses that forbid
// hipMalloc).  The kernels and the work are those of lynx_linear_sparse_lora.
#include <atomic>
#include <mutex>

#include "lynx_debug.h"
#include "lynx_internal.h"

namespace lynx {
namespace {

// One copy per device, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: the device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
__device__ __align__(256) char scratch[LYNX_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on the first call on it).
lynx_status scratch_of_current_device(char** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return LYNX_ERR_DEVICE;
    }
    char* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            void* addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess ||
                addr == nullptr) {
                (void)hipGetLastError();
                return LYNX_ERR_DEVICE;
            }
            p = static_cast<char*>(addr);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LYNX_OK;
}

}  // namespace
}  // namespace lynx

using namespace lynx;

extern "C" lynx_status lynx_linear_sparse_lora_noalloc(const uint16_t* X, const uint16_t* W,
                                                       const uint16_t* LA, const uint16_t* LB,
                                                       uint16_t* Y, int64_t M, int64_t N,
                                                       int64_t K, int64_t R,
                                                       lynx_stream_t stream) {
    bool noop = false;
    lynx_status st = validate_sparse_layer(X, W, LA, LB, Y, M, N, K, R, &noop);
    if (st != LYNX_OK || noop) return st;
    // K1 writes every byte of the packed operand (padding rows included), s
    // and T that K2 reads, so nothing in the array needs clearing
    if (sparse_workspace_bytes(M, K, R) > LYNX_SCRATCH_BYTES) return LYNX_ERR_SCRATCH;
    st = check_device();
    if (st != LYNX_OK) return st;
    char* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != LYNX_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return debug_sync(run_sparse_layer(X, W, LA, LB, Y, M, N, K, R, ws, s), s);
}
