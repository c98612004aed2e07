"""The library from plain C: tests/c_abi/lynx_c_example.c links only
liblynx.so and the HIP runtime, allocates with hipMalloc and calls
lynx_linear_sparse_lora and lynx_linear_dense through include/lynx.h.

On the GPU, its Y must be the same bytes as the same calls made through the
Python binding (the same kernels), and within the parity bar of the oracle.
On the CPU, its argument and file errors exit with the documented statuses
before any HIP call.
"""
import os

import numpy as np
import pytest
import torch

import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.c_abi import c_example
from tests.gpu_util import dev, say
from workloads import make_layer

needs_binary = pytest.mark.skipif(not os.path.exists(c_example.BIN),
                                  reason="tests/c_abi/lynx_c_example is not built (__graft_entry__.build())")


@needs_binary
def test_c_example_argument_and_file_errors(tmp_path):
    res = c_example.run([])
    assert res.returncode == 2 and "usage" in res.stderr
    res = c_example.run([tmp_path, 16, 16, 64, -1])
    assert res.returncode == 2
    res = c_example.run([tmp_path, 16, 16, 64, 0])   # no X.bin there
    assert res.returncode == 3 and "X.bin" in res.stderr


@needs_binary
@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N,R", [(1024, 512, 1024, 64),    # tiled kernels
                                     (100, 640, 130, 48),      # 64 x 64 kernels, ragged
                                     (300, 1152, 257, 0)])     # no LoRA, N % 8 != 0
def test_c_example_matches_the_binding_and_the_oracle(tmp_path, M, K, N, R):
    L = make_layer(M, K, N, "heavy", seed=M + 17, R=max(R, 16))
    files = {"X.bin": L.X, "W.bin": L.W}
    if R > 0:
        files.update({"LA.bin": L.LA, "LB.bin": L.LB})
    for name, bits in files.items():
        np.ascontiguousarray(bits, dtype="<u2").tofile(tmp_path / name)
    say(f"C example M={M} K={K} N={N} R={R}")
    res = c_example.run([tmp_path, M, N, K, R])
    assert res.returncode == 0, res.stderr
    y_sparse = np.fromfile(tmp_path / "Y_sparse.bin", dtype="<u2").reshape(M, N)
    y_dense = np.fromfile(tmp_path / "Y_dense.bin", dtype="<u2").reshape(M, N)

    LA, LB = (None, None) if R == 0 else (L.LA, L.LB)
    Ys = gu.sparse_lora(dev(L.X), dev(L.W), None if R == 0 else dev(LA), None if R == 0 else dev(LB))
    Yd = gu.dense(dev(L.X), dev(L.W))
    torch.cuda.synchronize()
    assert np.array_equal(y_sparse, gu.host_bits(Ys)), "C and Python calls of the sparse layer differ"
    assert np.array_equal(y_dense, gu.host_bits(Yd)), "C and Python calls of the dense layer differ"
    from tests.test_gpu_linear import check
    as_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)  # noqa: E731
    check(as_bf16(y_sparse), orc.linear_sparse_lora(L.X, L.W, LA, LB), f"C sparse_lora {M}x{K}->{N}")
    check(as_bf16(y_dense), orc.linear_dense(L.X, L.W), f"C dense {M}x{K}->{N}")
