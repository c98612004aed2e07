// C ABI of liblynx: argument validation, workspace layout and dispatch.
// The operations themselves are defined in lynx.h; the kernels live in the
// other translation units.
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "lynx_debug.h"
#include "lynx_internal.h"

namespace lynx {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cu_count[kMaxDevices];    // 0 unknown

constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxElems = int64_t(1) << 31;
// The tiled GEMMs address every operand with unsigned 32-bit byte offsets
// through buffer resources, including the rows and columns of a last partial
// 256-wide tile that lie past the tensor (the range check drops them); with
// the dimensions padded by one tile the tensors stay below 2^31 elements, so
// those offsets stay below 2^32 and never wrap into the tensor.
constexpr int64_t kPad = 256;

inline size_t round_up256(size_t x) { return (x + 255) & ~size_t(255); }

bool rank_ok(int64_t R) { return R == 0 || R == 16 || R == 32 || R == 48 || R == 64; }

bool dims_ok(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0) return false;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return false;
    if (K % 64 != 0) return false;
    if ((M + kPad) * K >= kMaxElems || (N + kPad) * K >= kMaxElems || (M + kPad) * N >= kMaxElems)
        return false;
    return true;
}

struct WorkspaceLayout {
    size_t values, meta, scale, T, total;
};

WorkspaceLayout layout_for(int64_t M, int64_t K, int64_t R) {
    const size_t Mp = size_t((M + 15) / 16) * 16;  // packed operand rows, whole 16-row tiles
    WorkspaceLayout L;
    L.values = 0;
    L.meta = L.values + round_up256(Mp * size_t(K / 2) * 2);
    L.scale = L.meta + round_up256(Mp * size_t(K / 8));
    L.T = L.scale + round_up256(size_t(M) * 4);
    L.total = L.T + round_up256(size_t(M) * size_t(R) * 2);
    return L;
}
}  // namespace

lynx_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LYNX_ERR_UNSUPPORTED_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return LYNX_ERR_UNSUPPORTED_DEVICE;
    int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return LYNX_ERR_DEVICE;
        }
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? LYNX_OK : LYNX_ERR_UNSUPPORTED_DEVICE;
}

lynx_status device_cu_count(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return LYNX_ERR_DEVICE;
    }
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            return LYNX_ERR_DEVICE;
        }
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    *cus = n;
    return LYNX_OK;
}

}  // namespace lynx

namespace lynx {
lynx_status validate_sparse_layer(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                                  const uint16_t* LB, const uint16_t* Y, int64_t M, int64_t N,
                                  int64_t K, int64_t R, bool* noop) {
    *noop = false;
    if (!dims_ok(M, N, K) || !rank_ok(R)) return LYNX_ERR_SHAPE;
    if (M == 0 || N == 0) {
        *noop = true;
        return LYNX_OK;
    }
    if (!X || !W || !Y) return LYNX_ERR_NULL;
    if (R > 0 && (!LA || !LB)) return LYNX_ERR_NULL;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return LYNX_ERR_ALIGN;
    if (R > 0 && (!aligned16(LA) || !aligned16(LB))) return LYNX_ERR_ALIGN;
    return LYNX_OK;
}

size_t sparse_workspace_bytes(int64_t M, int64_t K, int64_t R) {
    return layout_for(M, K, R).total;
}

lynx_status debug_sync(lynx_status st, hipStream_t stream) {
    if (st != LYNX_OK) return st;
    const char* v = std::getenv("LYNX_DEBUG");
    if (!v || !*v || std::strcmp(v, "0") == 0) return st;
    // no wait on a stream under capture, nor when the query itself fails (as
    // it can for the legacy stream while another stream captures globally)
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return st;
    }
    if (cs != hipStreamCaptureStatusNone) return st;
    if (hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return LYNX_ERR_DEVICE;
    }
    return st;
}

// the sparse layer on validated arguments
lynx_status run_sparse_layer(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                             const uint16_t* LB, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                             int64_t R, void* workspace, hipStream_t s) {
    const WorkspaceLayout L = layout_for(M, K, R);
    char* ws = static_cast<char*>(workspace);
    uint16_t* values = reinterpret_cast<uint16_t*>(ws + L.values);
    uint8_t* meta = reinterpret_cast<uint8_t*>(ws + L.meta);
    float* scale = reinterpret_cast<float*>(ws + L.scale);
    uint16_t* T = R > 0 ? reinterpret_cast<uint16_t*>(ws + L.T) : nullptr;
    lynx_status st = launch_sparsify(X, R > 0 ? LB : nullptr, int(M), int(K), int(R), values,
                                     meta, scale, T, s);
    if (st != LYNX_OK) return st;
    return launch_gemm_sparse(values, meta, scale, T, W, R > 0 ? LA : nullptr, Y, int(M), int(N),
                              int(K), int(R), s);
}
}  // namespace lynx

using namespace lynx;

extern "C" {

const char* lynx_status_string(lynx_status s) {
    switch (s) {
        case LYNX_OK: return "LYNX_OK";
        case LYNX_ERR_NULL: return "LYNX_ERR_NULL: a required pointer is NULL";
        case LYNX_ERR_SHAPE: return "LYNX_ERR_SHAPE: a size is outside the supported limits";
        case LYNX_ERR_ALIGN: return "LYNX_ERR_ALIGN: a pointer is not 16-byte aligned";
        case LYNX_ERR_WORKSPACE: return "LYNX_ERR_WORKSPACE: workspace is NULL or too small";
        case LYNX_ERR_DEVICE: return "LYNX_ERR_DEVICE: a HIP call or kernel launch failed";
        case LYNX_ERR_UNSUPPORTED_DEVICE:
            return "LYNX_ERR_UNSUPPORTED_DEVICE: the current device is not gfx950";
        case LYNX_ERR_SCRATCH:
            return "LYNX_ERR_SCRATCH: the problem needs more workspace than the library's "
                   "static scratch array holds (64 MiB); call lynx_linear_sparse_lora with a "
                   "workspace instead";
    }
    return "LYNX_ERR_UNKNOWN";
}

int lynx_version(void) { return 100; }

size_t lynx_workspace_bytes(int64_t M, int64_t K, int64_t R) {
    if (!dims_ok(M, 1, K) || !rank_ok(R)) return 0;
    return layout_for(M, K, R).total;
}

lynx_status lynx_sparsify(const uint16_t* X, const uint16_t* LB, int64_t M, int64_t K, int64_t R,
                          uint16_t* values, uint8_t* meta, float* scale, uint16_t* T,
                          lynx_stream_t stream) {
    if (!dims_ok(M, 1, K) || !rank_ok(R)) return LYNX_ERR_SHAPE;
    if (M == 0) return LYNX_OK;
    if (!X || !values || !meta || !scale) return LYNX_ERR_NULL;
    if (R > 0 && (!LB || !T)) return LYNX_ERR_NULL;
    if (!aligned16(X) || !aligned16(values) || !aligned16(meta) || !aligned16(scale))
        return LYNX_ERR_ALIGN;
    if (R > 0 && (!aligned16(LB) || !aligned16(T))) return LYNX_ERR_ALIGN;
    lynx_status st = check_device();
    if (st != LYNX_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return debug_sync(launch_sparsify(X, R > 0 ? LB : nullptr, int(M), int(K), int(R), values,
                                      meta, scale, R > 0 ? T : nullptr, s),
                      s);
}

lynx_status lynx_linear_sparse_lora_packed(const uint16_t* values, const uint8_t* meta,
                                           const float* scale, const uint16_t* T,
                                           const uint16_t* W, const uint16_t* LA, uint16_t* Y,
                                           int64_t M, int64_t N, int64_t K, int64_t R,
                                           lynx_stream_t stream) {
    if (!dims_ok(M, N, K) || !rank_ok(R)) return LYNX_ERR_SHAPE;
    if (M == 0 || N == 0) return LYNX_OK;
    if (!values || !meta || !scale || !W || !Y) return LYNX_ERR_NULL;
    if (R > 0 && (!T || !LA)) return LYNX_ERR_NULL;
    if (!aligned16(values) || !aligned16(meta) || !aligned16(scale) || !aligned16(W) ||
        !aligned16(Y))
        return LYNX_ERR_ALIGN;
    if (R > 0 && (!aligned16(T) || !aligned16(LA))) return LYNX_ERR_ALIGN;
    lynx_status st = check_device();
    if (st != LYNX_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return debug_sync(launch_gemm_sparse(values, meta, scale, R > 0 ? T : nullptr, W,
                                         R > 0 ? LA : nullptr, Y, int(M), int(N), int(K), int(R), s),
                      s);
}


namespace {
// Argument checks of the sparse layer with a caller workspace; LYNX_OK with
// *noop set for M or N == 0.
lynx_status validate_sparse(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                            const uint16_t* LB, const uint16_t* Y, int64_t M, int64_t N,
                            int64_t K, int64_t R, const void* workspace, size_t workspace_bytes,
                            bool* noop) {
    lynx_status st = validate_sparse_layer(X, W, LA, LB, Y, M, N, K, R, noop);
    if (st != LYNX_OK || *noop) return st;
    if (!workspace || workspace_bytes < layout_for(M, K, R).total) return LYNX_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LYNX_ERR_ALIGN;
    return LYNX_OK;
}

lynx_status validate_dense(const uint16_t* X, const uint16_t* W, const uint16_t* Y, int64_t M,
                           int64_t N, int64_t K, bool* noop) {
    *noop = false;
    if (!dims_ok(M, N, K)) return LYNX_ERR_SHAPE;
    if (M == 0 || N == 0) {
        *noop = true;
        return LYNX_OK;
    }
    if (!X || !W || !Y) return LYNX_ERR_NULL;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return LYNX_ERR_ALIGN;
    return LYNX_OK;
}
}  // namespace

lynx_status lynx_linear_sparse_lora(const uint16_t* X, const uint16_t* W, const uint16_t* LA,
                                    const uint16_t* LB, uint16_t* Y, int64_t M, int64_t N,
                                    int64_t K, int64_t R, void* workspace,
                                    size_t workspace_bytes, lynx_stream_t stream) {
    bool noop = false;
    lynx_status st = validate_sparse(X, W, LA, LB, Y, M, N, K, R, workspace, workspace_bytes,
                                     &noop);
    if (st != LYNX_OK || noop) return st;
    st = check_device();
    if (st != LYNX_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return debug_sync(run_sparse_layer(X, W, LA, LB, Y, M, N, K, R, workspace, s), s);
}

lynx_status lynx_linear_dense(const uint16_t* X, const uint16_t* W, uint16_t* Y, int64_t M,
                              int64_t N, int64_t K, lynx_stream_t stream) {
    bool noop = false;
    lynx_status st = validate_dense(X, W, Y, M, N, K, &noop);
    if (st != LYNX_OK || noop) return st;
    st = check_device();
    if (st != LYNX_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return debug_sync(launch_gemm_dense(X, W, Y, int(M), int(N), int(K), s), s);
}

size_t lynx_sequence_workspace_bytes(const lynx_layer* layers, int64_t n) {
    if (n < 0 || (n > 0 && !layers)) return 0;
    size_t need = 0;
    for (int64_t i = 0; i < n; ++i) {
        const lynx_layer& L = layers[i];
        if (L.mode == LYNX_LAYER_DENSE) {
            if (!dims_ok(L.M, L.N, L.K)) return 0;
        } else if (L.mode == LYNX_LAYER_SPARSE_LORA) {
            if (!dims_ok(L.M, L.N, L.K) || !rank_ok(L.R)) return 0;
            if (L.M > 0 && L.N > 0) {
                const size_t b = layout_for(L.M, L.K, L.R).total;
                if (b > need) need = b;
            }
        } else {
            return 0;
        }
    }
    return need;
}

lynx_status lynx_linear_sequence(const lynx_layer* layers, int64_t n, void* workspace,
                                 size_t workspace_bytes, lynx_stream_t stream) {
    if (n < 0) return LYNX_ERR_SHAPE;
    if (n == 0) return LYNX_OK;
    if (!layers) return LYNX_ERR_NULL;
    bool any = false;
    for (int64_t i = 0; i < n; ++i) {
        const lynx_layer& L = layers[i];
        bool noop = false;
        lynx_status st;
        if (L.mode == LYNX_LAYER_DENSE) {
            st = validate_dense(L.X, L.W, L.Y, L.M, L.N, L.K, &noop);
        } else if (L.mode == LYNX_LAYER_SPARSE_LORA) {
            st = validate_sparse(L.X, L.W, L.LA, L.LB, L.Y, L.M, L.N, L.K, L.R, workspace,
                                 workspace_bytes, &noop);
        } else {
            st = LYNX_ERR_SHAPE;
        }
        if (st != LYNX_OK) return st;
        any = any || !noop;
    }
    if (!any) return LYNX_OK;
    lynx_status st = check_device();
    if (st != LYNX_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int64_t i = 0; i < n; ++i) {
        const lynx_layer& L = layers[i];
        if (L.M == 0 || L.N == 0) continue;
        if (L.mode == LYNX_LAYER_DENSE) {
            st = launch_gemm_dense(L.X, L.W, L.Y, int(L.M), int(L.N), int(L.K), s);
        } else {
            st = run_sparse_layer(L.X, L.W, L.LA, L.LB, L.Y, L.M, L.N, L.K, L.R, workspace, s);
        }
        if (st != LYNX_OK) return st;
    }
    return debug_sync(LYNX_OK, s);
}

}  // extern "C"
