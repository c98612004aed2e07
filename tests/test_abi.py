"""The C ABI: the library loads, exports every symbol the headers declare, and
rejects bad arguments with the documented status before touching a device.

No call here reaches a kernel launch: every argument set fails validation (or
is a documented no-op) before the device is queried.
"""
import ctypes
import glob
import os
import re

import pytest

from activation_sparse_gemm_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, WORKSPACE, DEVICE, UNSUPPORTED, SCRATCH = range(8)

A = 0x10000  # a fake, 16-byte-aligned address: validation fails before any use
B = 0x20000


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(lynx_\w+)\s*\(", text))
    return names


def test_headers_declare_the_boundary():
    names = declared_functions()
    for required in ("lynx_sparsify", "lynx_linear_sparse_lora", "lynx_linear_sparse_lora_packed",
                     "lynx_linear_dense", "lynx_workspace_bytes", "lynx_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in _abi.SIGNATURES, f"binding lacks {name}"


def test_status_strings():
    for s in range(8):
        assert _abi.status_string(s).startswith(_abi.STATUS_NAMES[s])
    assert "UNKNOWN" in _abi.status_string(99)


def test_workspace_bytes():
    ws = _abi.workspace_bytes(4096, 3072, 64)
    # values M*K + meta M*K/8 + scale 4M + T 2MR, each 256-aligned
    assert ws == 4096 * 3072 + 4096 * 3072 // 8 + 4096 * 4 + 4096 * 64 * 2
    # M = 3 -> 16 stored rows: values 16*128 B, meta 16*16 B, scale and T rounded to 256 B
    assert _abi.workspace_bytes(3, 128, 16) == 2048 + 256 + 256 + 256
    assert _abi.workspace_bytes(16, 100, 0) == 0      # K not a multiple of 64
    assert _abi.workspace_bytes(16, 96, 0) == 0
    assert _abi.workspace_bytes(16, 64, 0) > 0       # K % 64 == 0 is enough
    assert _abi.workspace_bytes(16, 192, 16) > 0
    assert _abi.workspace_bytes(16, 128, 8) == 0      # unsupported rank
    assert _abi.workspace_bytes(-1, 128, 0) == 0


def call_sparsify(X=A, LB=A, M=16, K=128, R=16, values=A, meta=A, scale=A, T=A):
    return _abi.lib().lynx_sparsify(X, LB, M, K, R, values, meta, scale, T, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), SHAPE), (dict(K=0), SHAPE), (dict(K=96), SHAPE), (dict(M=-1), SHAPE),
    (dict(R=8), SHAPE), (dict(R=80), SHAPE), (dict(M=1 << 25), SHAPE),
    (dict(X=None), NULL), (dict(values=None), NULL), (dict(meta=None), NULL),
    (dict(scale=None), NULL), (dict(LB=None), NULL), (dict(T=None), NULL),
    (dict(X=A + 2), ALIGN), (dict(meta=A + 8), ALIGN), (dict(T=A + 4), ALIGN),
    (dict(M=0), OK),
])
def test_sparsify_validation(kw, status):
    assert call_sparsify(**kw) == status


def call_linear(X=A, W=A, LA=A, LB=A, Y=A, M=16, N=16, K=128, R=16, ws=B, wsb=1 << 20):
    return _abi.lib().lynx_linear_sparse_lora(X, W, LA, LB, Y, M, N, K, R, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=160), SHAPE), (dict(N=-3), SHAPE), (dict(R=17), SHAPE),
    (dict(W=None), NULL), (dict(LA=None), NULL), (dict(Y=None), NULL),
    (dict(Y=A + 2), ALIGN), (dict(ws=B + 16), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE),
    (dict(N=0), OK), (dict(M=0), OK),
])
def test_linear_validation(kw, status):
    assert call_linear(**kw) == status


def test_linear_workspace_exact_boundary():
    need = _abi.workspace_bytes(16, 128, 16)
    assert call_linear(wsb=need - 1) == WORKSPACE


def call_noalloc(X=A, W=A, LA=A, LB=A, Y=A, M=16, N=16, K=128, R=16):
    return _abi.lib().lynx_linear_sparse_lora_noalloc(X, W, LA, LB, Y, M, N, K, R, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=160), SHAPE), (dict(R=17), SHAPE), (dict(M=1 << 25), SHAPE),
    (dict(W=None), NULL), (dict(LB=None), NULL), (dict(Y=A + 2), ALIGN),
    (dict(M=0), OK), (dict(N=0), OK),
    # the static scratch array holds LYNX_SCRATCH_BYTES = 64 MiB
    (dict(M=9216, K=12288, R=64), SCRATCH), (dict(M=8192, K=8192, R=0), SCRATCH),
])
def test_noalloc_validation(kw, status):
    assert call_noalloc(**kw) == status


def test_noalloc_scratch_limit_is_the_workspace_size():
    """A problem is accepted exactly when its workspace fits the array."""
    import torch
    fits = [(4096, 12288, 64), (4096, 3072, 64), (7248, 8192, 16), (9520, 6144, 64)]
    too_big = [(9216, 12288, 64), (7249, 8192, 16), (9521, 6144, 64)]
    for M, K, R in fits:
        assert 0 < _abi.workspace_bytes(M, K, R) <= _abi.SCRATCH_BYTES
    for M, K, R in too_big:
        assert _abi.workspace_bytes(M, K, R) > _abi.SCRATCH_BYTES
        assert call_noalloc(M=M, K=K, R=R) == SCRATCH
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid fake pointers must not reach a launch")
    for M, K, R in fits:
        assert call_noalloc(M=M, K=K, R=R) == UNSUPPORTED


def call_packed(v=A, m=A, s=A, T=A, W=A, LA=A, Y=A, M=16, N=16, K=128, R=16):
    return _abi.lib().lynx_linear_sparse_lora_packed(v, m, s, T, W, LA, Y, M, N, K, R, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=1), SHAPE), (dict(R=100), SHAPE), (dict(v=None), NULL), (dict(T=None), NULL),
    (dict(s=A + 4), ALIGN), (dict(LA=A + 2), ALIGN), (dict(M=0), OK),
])
def test_packed_validation(kw, status):
    assert call_packed(**kw) == status


@pytest.mark.parametrize("args,status", [
    ((A, A, A, 16, 16, 96), SHAPE), ((None, A, A, 16, 16, 128), NULL),
    ((A, A, A + 6, 16, 16, 128), ALIGN), ((A, A, A, 0, 16, 128), OK),
])
def test_dense_validation(args, status):
    assert _abi.lib().lynx_linear_dense(*args, None) == status


@pytest.mark.parametrize("K,ok", [(32, False), (96, False), (160, False), (64, True), (192, True),
                                  (320, True)])
def test_k_must_be_a_multiple_of_64(K, ok):
    """K % 64 == 0 passes validation (without a GPU the call then stops at the
    device check); anything else is LYNX_ERR_SHAPE for every entry point."""
    import torch
    if ok and torch.cuda.is_available():
        pytest.skip("a GPU is present: valid fake pointers must not reach a launch")
    want = UNSUPPORTED if ok else SHAPE
    assert call_linear(K=K) == want
    assert call_packed(K=K) == want
    assert call_sparsify(K=K) == want
    assert call_noalloc(K=K) == want
    assert _abi.lib().lynx_linear_dense(A, A, A, 16, 16, K, None) == want


# The tiled kernels address every operand with unsigned 32-bit byte offsets,
# padded rows and columns of a partial 256-wide tile included: (M + 256) K,
# (N + 256) K and (M + 256) N must each stay below 2^31 elements.
LIMIT = 1 << 31


@pytest.mark.parametrize("M,N,K", [
    (LIMIT // 16384 - 256, 16, 16384),      # (M + 256) K == 2^31
    (16, LIMIT // 16384 - 256, 16384),      # (N + 256) K == 2^31
    ((1 << 20) - 256, 2048, 128),           # (M + 256) N == 2^31
])
def test_shape_limit_of_32bit_offsets_rejects(M, N, K):
    lib = _abi.lib()
    assert call_linear(M=M, N=N, K=K) == SHAPE
    assert call_packed(M=M, N=N, K=K) == SHAPE
    assert lib.lynx_linear_dense(A, A, A, M, N, K, None) == SHAPE
    assert call_sequence(layers_of((M, N, K, 16, SP))) == SHAPE
    if (M + 256) * K >= LIMIT:
        assert call_sparsify(M=M, K=K) == SHAPE
        assert _abi.workspace_bytes(M, K, 16) == 0


@pytest.mark.parametrize("M,N,K", [
    (LIMIT // 16384 - 257, 16, 16384), (16, LIMIT // 16384 - 257, 16384),
    ((1 << 20) - 256, 2047, 128),
])
def test_shape_limit_of_32bit_offsets_admits(M, N, K):
    """One row or column below the limit passes validation: without a GPU the
    call stops at the device check (it never launches)."""
    import torch
    assert _abi.workspace_bytes(M, K, 16) > 0
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid fake pointers must not reach a launch")
    assert call_linear(M=M, N=N, K=K, wsb=1 << 40) == UNSUPPORTED
    assert call_packed(M=M, N=N, K=K) == UNSUPPORTED
    assert _abi.lib().lynx_linear_dense(A, A, A, M, N, K, None) == UNSUPPORTED
    assert call_sparsify(M=M, K=K) == UNSUPPORTED


def test_probe_validation():
    L = _abi.lib()
    assert L.lynx_probe_mfma(4, 0, A, A, A, A, None) == SHAPE
    assert L.lynx_probe_mfma(0, 2, A, A, A, A, None) == SHAPE
    assert L.lynx_probe_mfma(0, 0, A, A, None, A, None) == NULL
    assert L.lynx_probe_mfma(1, 0, A + 1, A, A, A, None) == ALIGN
    assert L.lynx_probe_mfma_rate(4, 16, 256, A, B, None) == SHAPE
    assert L.lynx_probe_mfma_rate(0, 0, 256, A, B, None) == SHAPE
    assert L.lynx_probe_mfma_rate(0, 16, 0, A, B, None) == SHAPE
    assert L.lynx_probe_mfma_rate(1, 16, 256, None, B, None) == NULL
    assert L.lynx_probe_mfma_rate(1, 16, 256, A, B + 8, None) == ALIGN


def test_valid_arguments_without_gpu_report_unsupported_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid fake pointers must not reach a launch")
    assert call_sparsify() == UNSUPPORTED
    assert call_linear() == UNSUPPORTED


@pytest.mark.parametrize("value", ["1", "0", ""])
def test_debug_mode_leaves_validation_unchanged(monkeypatch, value):
    """LYNX_DEBUG only adds a wait after work was queued: every argument error,
    every no-op and the device check come out as without it."""
    monkeypatch.setenv("LYNX_DEBUG", value)
    assert call_sparsify(K=100) == SHAPE and call_sparsify(X=None) == NULL
    assert call_sparsify(M=0) == OK
    assert call_linear(wsb=100) == WORKSPACE and call_linear(N=0) == OK
    assert _abi.lib().lynx_linear_sequence(None, 0, B, 1 << 20, None) == OK
    import torch
    if not torch.cuda.is_available():
        assert call_sparsify() == UNSUPPORTED and call_linear() == UNSUPPORTED


def test_binding_raises_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _abi.lib()


def layers_of(*specs):
    """ctypes array of lynx_layer from (M, N, K, R, mode) tuples with fake pointers."""
    arr = (_abi.Layer * len(specs))()
    for i, (M, N, K, R, mode) in enumerate(specs):
        arr[i] = _abi.Layer(A, A, A if R else None, A if R else None, B, M, N, K, R, mode)
    return arr


SP, DN = _abi.LAYER_SPARSE_LORA, _abi.LAYER_DENSE


def test_sequence_workspace_bytes_is_the_largest_sparse_layer():
    arr = layers_of((9216, 9216, 3072, 64, SP), (9216, 3072, 3072, 64, DN),
                    (9216, 12288, 3072, 64, SP), (9216, 3072, 12288, 64, SP))
    want = max(_abi.workspace_bytes(9216, 3072, 64), _abi.workspace_bytes(9216, 12288, 64))
    assert _abi.lib().lynx_sequence_workspace_bytes(arr, 4) == want
    assert _abi.lib().lynx_sequence_workspace_bytes(layers_of((16, 16, 128, 0, DN)), 1) == 0
    assert _abi.lib().lynx_sequence_workspace_bytes(layers_of((16, 16, 100, 0, DN)), 1) == 0
    assert _abi.lib().lynx_sequence_workspace_bytes(layers_of((16, 16, 128, 0, 7)), 1) == 0


def call_sequence(arr, n=None, ws=B, wsb=1 << 30):
    return _abi.lib().lynx_linear_sequence(arr, len(arr) if n is None else n, ws, wsb, None)


def test_sequence_validation():
    good = (16, 16, 128, 16, SP)
    assert call_sequence(layers_of(good), n=0) == OK
    assert _abi.lib().lynx_linear_sequence(None, 2, B, 1 << 20, None) == NULL
    assert call_sequence(layers_of(good), n=-1) == SHAPE
    # the first failing layer's status, whatever the others are
    assert call_sequence(layers_of(good, (16, 16, 96, 16, SP))) == SHAPE
    assert call_sequence(layers_of(good, (16, 16, 128, 0, 5))) == SHAPE
    assert call_sequence(layers_of((16, 16, 128, 16, SP)), ws=None) == WORKSPACE
    assert call_sequence(layers_of(good), wsb=_abi.workspace_bytes(16, 128, 16) - 1) == WORKSPACE
    assert call_sequence(layers_of(good), ws=B + 16) == ALIGN
    arr = layers_of(good, (16, 16, 128, 0, DN))
    arr[1].X = A + 2
    assert call_sequence(arr) == ALIGN
    arr = layers_of(good)
    arr[0].LA = None
    assert call_sequence(arr) == NULL
    # empty layers are no-ops and need no device
    assert call_sequence(layers_of((0, 16, 128, 16, SP), (16, 0, 128, 0, DN)), ws=None) == OK


def test_sequence_without_gpu_reports_unsupported_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid fake pointers must not reach a launch")
    # a dense-only sequence needs no workspace
    assert call_sequence(layers_of((16, 16, 128, 0, DN)), ws=None) == UNSUPPORTED
    assert call_sequence(layers_of((16, 16, 128, 16, SP), (16, 16, 128, 0, DN))) == UNSUPPORTED
