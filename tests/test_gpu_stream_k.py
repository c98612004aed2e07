"""The sparse GEMM with tiles split along K over the compute units (stream-K),
against the oracle and against itself.

The layer's schedule (lynx_probe_sparse_plan) splits these shapes: every
tile at 4096 x 512 -> 4352 (two-tile ranges, one partial sum per tile), the
same with ragged M and N (edge tiles among the split ones), every tile at the
MLP-down shape 4096 x 12288 -> 3072 (one-tile ranges: owners add two partial
sums), and the block's attention-out layer 9216 x 3072 -> 3072.  Each test
first asserts that the plan on this device does split the shape.

Bars: per-row relative Frobenius error <= 5e-3 against the fp64 oracle (all
rows of the small shapes, sampled rows plus the rows of split tiles' edges at
full size); two calls with differently poisoned workspaces give the same bits
(partial sums are added in a fixed order whatever arrives first); the GEMM
alone with the same schedule (lynx_probe_gemm_sparse_ws) gives the layer's
bits; the whole-tile schedule of the packed entry point agrees within the bar.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from activation_sparse_gemm_amd import _abi
from oracle import lynx_oracle as orc
from tests.gpu_util import ROW_REL_TOL, dev, host_f64, report, row_rel_err, sample_rows, say
from workloads import make_layer

pytestmark = pytest.mark.gpu

CASES = [  # M, K, N, R, rows checked against the oracle
    (4096, 512, 4352, 64, "all"),
    (4000, 512, 4300, 32, "all"),
    (4096, 512, 4352, 0, "all"),
    (4096, 12288, 3072, 64, "sampled"),
    (9216, 3072, 3072, 64, "sampled"),
]


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def rows_for(M, how):
    if how == "all":
        return np.arange(M)
    # sampled rows plus the first and last rows of every 256-row tile
    edges = np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256)])
    return np.unique(np.concatenate([sample_rows(M, n=40, seed=M), edges[edges < M]]))


@pytest.mark.parametrize("M,K,N,R,how", CASES)
def test_stream_k_layer_matches_oracle(M, K, N, R, how):
    plan = _abi.sparse_plan(M, N, K, True, cus())
    assert plan["sk_tiles"] > 0, plan
    L = make_layer(M, K, N, "heavy" if K < 12288 else "gelu", seed=M + N + R, R=max(R, 16))
    LA, LB = (None, None) if R == 0 else (L.LA, L.LB)
    say(f"stream-K layer M={M} K={K} N={N} R={R} plan={plan}")
    Y = gu.sparse_lora(dev(L.X), dev(L.W), None if R == 0 else dev(LA), None if R == 0 else dev(LB))
    torch.cuda.synchronize()
    rows = rows_for(M, how)
    Yg = host_f64(Y)[rows]
    ref = orc.linear_sparse_lora(L.X[rows], L.W, LA, LB)
    rep = report(f"stream-K {M}x{K}->{N} R{R}", Yg, ref)
    assert rep["nonfinite"] == 0 and rep["max_row_rel"] <= ROW_REL_TOL


@pytest.mark.parametrize("M,K,N,R", [(4096, 512, 4352, 64), (4096, 12288, 3072, 64)])
def test_stream_k_is_deterministic_and_matches_the_gemm_hook(M, K, N, R):
    assert _abi.sparse_plan(M, N, K, True, cus())["sk_tiles"] > 0
    L = make_layer(M, K, N, "heavy", seed=7, R=R)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    nbytes = lynx.workspace_bytes(M, N, K, R)
    outs = []
    for fill in (0x00, 0xFF, 0x5A):
        say(f"stream-K determinism M={M} K={K} N={N} workspace fill {fill:#x}")
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        Y = gu.nan_bf16((M, N))
        lynx.linear_sparse_lora(X, W, LA, LB, Y=Y, workspace=ws)
        torch.cuda.synchronize()
        outs.append(Y.view(torch.int16).clone())
        del ws
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    # the GEMM alone, same schedule, on the packed operand
    v, m, s, T = gu.sparsify(X, LB)
    ws = torch.full((nbytes,), 0x77, dtype=torch.uint8, device="cuda")
    Yh = gu.nan_bf16((M, N))
    say(f"stream-K GEMM hook M={M} K={K} N={N}")
    _abi.linear_sparse_lora_packed_ws(v, m, s, T, W, LA, ws, Y=Yh)
    Yp = gu.packed(v, m, s, T, W, LA)   # whole tiles only
    torch.cuda.synchronize()
    assert torch.equal(Yh.view(torch.int16), outs[0]), "GEMM hook differs from the layer"
    err = row_rel_err(host_f64(Yp), host_f64(Yh))
    say(f"stream-K vs whole tiles: max row-rel {err.max():.3e}, "
        f"bit-identical fraction {float((Yp.view(torch.int16) == Yh.view(torch.int16)).float().mean()):.4f}")
    assert err.max() <= ROW_REL_TOL
