"""ctypes binding of liblynx.so (include/lynx.h, include/lynx_probe.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their data pointers and torch's current HIP stream are passed
to the C entry points.  Every computation runs in the library's HIP kernels;
there is no fallback.  If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblynx.so")

LYNX_OK = 0
STATUS_NAMES = {
    0: "LYNX_OK", 1: "LYNX_ERR_NULL", 2: "LYNX_ERR_SHAPE", 3: "LYNX_ERR_ALIGN",
    4: "LYNX_ERR_WORKSPACE", 5: "LYNX_ERR_DEVICE", 6: "LYNX_ERR_UNSUPPORTED_DEVICE",
    7: "LYNX_ERR_SCRATCH",
}
SCRATCH_BYTES = 64 << 20  # LYNX_SCRATCH_BYTES

LAYER_SPARSE_LORA, LAYER_DENSE = 0, 1


class Layer(ctypes.Structure):
    """struct lynx_layer (include/lynx.h)."""
    _fields_ = [("X", ctypes.c_void_p), ("W", ctypes.c_void_p), ("LA", ctypes.c_void_p),
                ("LB", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("R", ctypes.c_int64),
                ("mode", ctypes.c_int32)]


# every symbol the public headers declare, with (restype, argtypes)
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_LP = ctypes.POINTER(Layer)
SIGNATURES = {
    "lynx_status_string": (ctypes.c_char_p, [_I]),
    "lynx_version": (_I, []),
    "lynx_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "lynx_sparsify": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "lynx_linear_sparse_lora": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P]),
    "lynx_linear_sparse_lora_packed": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                            _P]),
    "lynx_linear_sparse_lora_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
    "lynx_linear_dense": (_I, [_P, _P, _P, _I64, _I64, _I64, _P]),
    "lynx_sequence_workspace_bytes": (_SZ, [_LP, _I64]),
    "lynx_linear_sequence": (_I, [_LP, _I64, _P, _SZ, _P]),
    "lynx_probe_mfma": (_I, [_I, _I, _P, _P, _P, _P, _P]),
    "lynx_probe_mfma_rate": (_I, [_I, _I, _I, _P, _P, _P]),
}


class LynxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m activation_sparse_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lynx_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != LYNX_OK:
        raise LynxError(status, where)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")


def version() -> int:
    return lib().lynx_version()


def workspace_bytes(M: int, K: int, R: int) -> int:
    return lib().lynx_workspace_bytes(M, K, R)


def padded_rows(M: int) -> int:
    """Rows of the stored packed operand: whole 16-row tiles."""
    return (M + 15) // 16 * 16


def sparsify(X: torch.Tensor, LB: torch.Tensor | None = None, out: dict | None = None):
    """Packed 2:4 operand and LoRA down-projection of X (lynx_sparsify).

    Returns (values, meta, scale, T): values (Mp*K/2,) bf16 and meta (Mp*K/8,)
    uint8 in the 16-row x 64-channel tile order of lynx.h (Mp = M rounded up
    to 16), scale [M] fp32, T [M, R] bf16 or None.
    """
    M, K = X.shape
    Mp = padded_rows(M)
    R = 0 if LB is None else LB.shape[0]
    _need(X, torch.bfloat16, (M, K), "X")
    if LB is not None:
        _need(LB, torch.bfloat16, (R, K), "LB")
    dev = X.device
    out = out or {}
    values = out.get("values")
    if values is None:
        values = torch.empty((Mp * K // 2,), dtype=torch.bfloat16, device=dev)
    meta = out.get("meta")
    if meta is None:
        meta = torch.empty((Mp * K // 8,), dtype=torch.uint8, device=dev)
    scale = out.get("scale")
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=dev)
    T = out.get("T")
    if T is None and R > 0:
        T = torch.empty((M, R), dtype=torch.bfloat16, device=dev)
    _need(values, torch.bfloat16, (Mp * K // 2,), "values")
    _need(meta, torch.uint8, (Mp * K // 8,), "meta")
    _need(scale, torch.float32, (M,), "scale")
    if R > 0:
        _need(T, torch.bfloat16, (M, R), "T")
    _check(lib().lynx_sparsify(_ptr(X), _ptr(LB), M, K, R, _ptr(values), _ptr(meta),
                               _ptr(scale), _ptr(T) if R > 0 else None, _stream(dev)),
           "lynx_sparsify")
    return values, meta, scale, (T if R > 0 else None)


def linear_sparse_lora(X, W, LA=None, LB=None, Y=None, workspace=None):
    """Y = S(X) W^T + X (LA LB)^T (lynx_linear_sparse_lora)."""
    M, K = X.shape
    N = W.shape[0]
    R = 0 if LA is None else LA.shape[1]
    _need(X, torch.bfloat16, (M, K), "X")
    _need(W, torch.bfloat16, (N, K), "W")
    if R > 0:
        _need(LA, torch.bfloat16, (N, R), "LA")
        _need(LB, torch.bfloat16, (R, K), "LB")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, N), "Y")
    nbytes = workspace_bytes(M, K, R)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=X.device)
    _check(lib().lynx_linear_sparse_lora(_ptr(X), _ptr(W), _ptr(LA), _ptr(LB), _ptr(Y), M, N, K,
                                         R, _ptr(workspace), workspace.numel(),
                                         _stream(X.device)),
           "lynx_linear_sparse_lora")
    return Y


def linear_sparse_lora_noalloc(X, W, LA=None, LB=None, Y=None):
    """Y = S(X) W^T + X (LA LB)^T with the library's static scratch array as
    workspace (lynx_linear_sparse_lora_noalloc): the C call allocates nothing.
    Pass Y to keep this wrapper from allocating it."""
    M, K = X.shape
    N = W.shape[0]
    R = 0 if LA is None else LA.shape[1]
    _need(X, torch.bfloat16, (M, K), "X")
    _need(W, torch.bfloat16, (N, K), "W")
    if R > 0:
        _need(LA, torch.bfloat16, (N, R), "LA")
        _need(LB, torch.bfloat16, (R, K), "LB")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, N), "Y")
    _check(lib().lynx_linear_sparse_lora_noalloc(_ptr(X), _ptr(W), _ptr(LA), _ptr(LB), _ptr(Y),
                                                 M, N, K, R, _stream(X.device)),
           "lynx_linear_sparse_lora_noalloc")
    return Y


def linear_sparse_lora_packed(values, meta, scale, T, W, LA=None, Y=None):
    """Y = scale * (X~ W^T) + T LA^T from a packed operand (lynx_linear_sparse_lora_packed)."""
    M = scale.shape[0]
    N, K = W.shape
    Mp = padded_rows(M)
    R = 0 if LA is None else LA.shape[1]
    _need(values, torch.bfloat16, (Mp * K // 2,), "values")
    _need(meta, torch.uint8, (Mp * K // 8,), "meta")
    _need(scale, torch.float32, (M,), "scale")
    _need(W, torch.bfloat16, (N, K), "W")
    if R > 0:
        _need(T, torch.bfloat16, (M, R), "T")
        _need(LA, torch.bfloat16, (N, R), "LA")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=W.device)
    _need(Y, torch.bfloat16, (M, N), "Y")
    _check(lib().lynx_linear_sparse_lora_packed(_ptr(values), _ptr(meta), _ptr(scale),
                                                _ptr(T) if R > 0 else None, _ptr(W),
                                                _ptr(LA) if R > 0 else None, _ptr(Y), M, N, K, R,
                                                _stream(W.device)),
           "lynx_linear_sparse_lora_packed")
    return Y


def linear_dense(X, W, Y=None):
    """Y = X W^T (lynx_linear_dense)."""
    M, K = X.shape
    N = W.shape[0]
    _need(X, torch.bfloat16, (M, K), "X")
    _need(W, torch.bfloat16, (N, K), "W")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, (M, N), "Y")
    _check(lib().lynx_linear_dense(_ptr(X), _ptr(W), _ptr(Y), M, N, K, _stream(X.device)),
           "lynx_linear_dense")
    return Y


def _layer_struct(d: dict) -> Layer:
    X, W, Y = d["X"], d["W"], d["Y"]
    M, K = X.shape
    N = W.shape[0]
    dense = d.get("dense", False)
    LA, LB = (None, None) if dense else (d.get("LA"), d.get("LB"))
    R = 0 if LA is None else LA.shape[1]
    _need(X, torch.bfloat16, (M, K), "X")
    _need(W, torch.bfloat16, (N, K), "W")
    _need(Y, torch.bfloat16, (M, N), "Y")
    if R > 0:
        _need(LA, torch.bfloat16, (N, R), "LA")
        _need(LB, torch.bfloat16, (R, K), "LB")
    return Layer(_ptr(X), _ptr(W), _ptr(LA), _ptr(LB), _ptr(Y), M, N, K, R,
                 LAYER_DENSE if dense else LAYER_SPARSE_LORA)


def sequence_workspace_bytes(layers: list) -> int:
    arr = (Layer * len(layers))(*[_layer_struct(d) for d in layers])
    return lib().lynx_sequence_workspace_bytes(arr, len(layers))


def linear_sequence(layers: list, workspace=None):
    """Runs the layers in order (lynx_linear_sequence).  Each layer is a dict
    with X, W, Y (device tensors), LA and LB for a sparse + LoRA layer, and
    dense=True for a skipped (dense) layer."""
    if not layers:
        return
    arr = (Layer * len(layers))(*[_layer_struct(d) for d in layers])
    dev = layers[0]["X"].device
    nbytes = lib().lynx_sequence_workspace_bytes(arr, len(layers))
    if workspace is None and nbytes > 0:
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    _check(lib().lynx_linear_sequence(arr, len(layers), _ptr(workspace),
                                      0 if workspace is None else workspace.numel(),
                                      _stream(dev)),
           "lynx_linear_sequence")


# dense-equivalent flops of one instruction of each probe kind: smfmac
# 16x16x64, smfmac 32x32x32, mfma 16x16x32, mfma 32x32x16 (bf16)
PROBE_NAMES = ("v_smfmac_f32_16x16x64_bf16", "v_smfmac_f32_32x32x32_bf16",
               "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_32x32x16_bf16")
PROBE_FLOPS = (2 * 16 * 16 * 64, 2 * 32 * 32 * 32, 2 * 16 * 16 * 32, 2 * 32 * 32 * 16)


def probe_mfma_rate(which: int, iters: int, grid: int, device=None) -> dict:
    """Runs lynx_probe_mfma_rate once on torch's current stream and returns the
    event-timed duration with the per-wave stamps (no arithmetic of the layer)."""
    dev = torch.device("cuda") if device is None else device
    sink = torch.empty((grid * 256,), dtype=torch.float32, device=dev)
    stamps = torch.zeros((grid * 4, 2), dtype=torch.int64, device=dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    _check(lib().lynx_probe_mfma_rate(which, iters, grid, _ptr(sink), _ptr(stamps), _stream(dev)),
           "lynx_probe_mfma_rate")
    end.record()
    torch.cuda.synchronize()
    return {"ms": start.elapsed_time(end), "stamps": stamps.cpu().numpy()}


def probe_mfma(which: int, abid: int, a: torch.Tensor, b: torch.Tensor,
               idx: torch.Tensor | None, d: torch.Tensor) -> torch.Tensor:
    """One matrix instruction per lane on raw register contents (lynx_probe_mfma)."""
    _check(lib().lynx_probe_mfma(which, abid, _ptr(a), _ptr(b), _ptr(idx), _ptr(d),
                                 _stream(a.device)),
           "lynx_probe_mfma")
    return d
