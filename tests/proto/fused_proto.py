"""Build, load and call the fused-sparsifier GEMM prototype
(k_fused_proto.hip): a measurement of the one-kernel design against the
library's sparsifier + sparse GEMM pair.  It is not part of the library and
nothing in the package calls it; bench.py --fusion-prototype times it and
tests/test_gpu_fused_proto.py checks it against the oracle.

    python -m tests.proto.fused_proto      # build libfused_proto.so
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "k_fused_proto.hip")
LIB_PATH = os.path.join(HERE, "libfused_proto.so")

_lib = None


def build(verbose: bool = True) -> str:
    """Compile the prototype for gfx950 with the library's own flags."""
    from activation_sparse_gemm_amd import build as _b
    tmp = LIB_PATH + ".tmp"
    cmd = [_b.HIPCC, *_b.COMMON, "-shared", SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {SRC}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tests.proto.fused_proto`")
        L = ctypes.CDLL(LIB_PATH)
        f = L.proto_gemm_fused
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
        _lib = L
    return _lib


def gemm_fused(X, W, Y=None):
    """Y [M x N] = s (X~ W^T) in one kernel, no LoRA term (bf16 tensors on the
    current device, row-major, contiguous).  Handles whole 256-row tiles,
    K % 128 == 0 and N a multiple of the tile width it picks (192 or 256);
    other shapes raise."""
    import torch
    assert X.dtype == W.dtype == torch.bfloat16 and X.is_cuda and W.is_cuda
    assert X.is_contiguous() and W.is_contiguous() and X.shape[1] == W.shape[1]
    M, K = X.shape
    N = W.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    assert Y.shape == (M, N) and Y.is_contiguous() and Y.dtype == torch.bfloat16
    stream = torch.cuda.current_stream(X.device).cuda_stream
    st = lib().proto_gemm_fused(X.data_ptr(), W.data_ptr(), Y.data_ptr(), M, N, K, stream)
    if st != 0:
        raise RuntimeError(f"proto_gemm_fused({M}, {N}, {K}): status {st}")
    return Y


if __name__ == "__main__":
    build()
