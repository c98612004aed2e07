"""Parity of the fused-sparsifier GEMM prototype (tests/proto) with the
oracle's layer without LoRA, s (X~ W^T): a 1024 x 512 -> 1536 problem whose
rows span s in [1, sqrt 2], checked whole, and the MLP-up and MLP-down shapes
on sampled rows.  The prototype is measured by bench.py --fusion-prototype; it
is not part of the library.

Bar: per-row relative Frobenius error <= 5e-3 against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from oracle import lynx_oracle as orc
from tests.gpu_util import ROW_REL_TOL, dev, host_f64, report, sample_rows, say
from tests.proto import fused_proto
from tests.test_gpu_edges import mixed_rows
from workloads import make_activation, make_weights

pytestmark = pytest.mark.gpu


def run(Xb, W):
    M, N = Xb.shape[0], W.shape[0]
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    fused_proto.gemm_fused(dev(Xb), dev(W), Y=Y)
    torch.cuda.synchronize()
    return host_f64(Y)


@pytest.mark.parametrize("M,K,N,kind", [(1024, 512, 1536, "mixed"), (4096, 3072, 12288, "heavy"),
                                        (4096, 12288, 3072, "gelu")])
def test_fused_prototype_matches_oracle(M, K, N, kind):
    Xb = mixed_rows(M, K, seed=41) if kind == "mixed" else make_activation(kind, M, K, seed=42)
    W = make_weights(N, K, 16, seed=43)[0]
    rows = np.arange(M) if M <= 1024 else sample_rows(M, n=48, seed=M)
    say(f"fused prototype: M={M} K={K} N={N} {kind}")
    Yg = run(Xb, W)[rows]
    Yref = orc.linear_sparse_lora(Xb[rows], W)
    rep = report(f"fused prototype {M}x{K}->{N}", Yg, Yref)
    assert rep["nonfinite"] == 0 and rep["max_row_rel"] <= ROW_REL_TOL


def test_fused_prototype_rejects_shapes_it_does_not_handle():
    X = torch.zeros((1000, 512), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((1536, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="status 2"):
        fused_proto.gemm_fused(X, W)
