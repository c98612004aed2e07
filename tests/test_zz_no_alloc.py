"""lynx_linear_sparse_lora_noalloc against lynx_linear_sparse_lora.

The no-allocation entry point runs the same kernels with its workspace in
the library's static scratch array: on the same inputs its Y must equal the
workspace entry point's bit for bit, and meet the oracle's 5e-3 per-row bar.
Two calls in a row, the second smaller, so the second runs on an array that
holds the first call's contents.  Sizes beyond the array are rejected
before any launch.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import ROW_REL_TOL, dev, host_f64, report, sample_rows, say
from workloads import make_layer

pytestmark = pytest.mark.gpu


def check_against_workspace_entry(M, K, N, R, seed):
    L = make_layer(M, K, N, "heavy", seed=seed, R=max(R, 16))
    X, W = dev(L.X), dev(L.W)
    LA, LB = (None, None) if R == 0 else (dev(L.LA), dev(L.LB))
    say(f"noalloc M={M} K={K} N={N} R={R}")
    Yn = gu.sparse_lora_noalloc(X, W, LA, LB)
    torch.cuda.synchronize()
    say(f"workspace entry M={M} K={K} N={N} R={R}")
    Yw = gu.sparse_lora(X, W, LA, LB)
    torch.cuda.synchronize()
    assert torch.equal(Yn.view(torch.int16), Yw.view(torch.int16)), "Y differs from the workspace entry"
    rows = sample_rows(M, n=24, seed=seed)
    Yg = host_f64(Yn)[rows]
    ref = orc.linear_sparse_lora(L.X[rows], L.W, None if R == 0 else L.LA, None if R == 0 else L.LB)
    rep = report(f"noalloc {M}x{K}->{N} R{R}", Yg, ref)
    assert rep["nonfinite"] == 0 and rep["max_row_rel"] <= ROW_REL_TOL


def test_noalloc_two_calls_second_smaller():
    # the MLP-up layer (14.7 MB of scratch), then a smaller ragged one that
    # runs the 192-wide tiles, then one small enough for the 64 x 64 kernels
    check_against_workspace_entry(4096, 3072, 12288, 64, seed=1)
    check_against_workspace_entry(1000, 640, 1100, 48, seed=2)
    check_against_workspace_entry(100, 256, 130, 0, seed=3)


def test_noalloc_rejects_problems_beyond_the_array():
    X = torch.zeros((9216, 12288), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((16, 12288), dtype=torch.bfloat16, device="cuda")
    LA = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    LB = torch.zeros((64, 12288), dtype=torch.bfloat16, device="cuda")
    assert lynx.workspace_bytes(9216, 12288, 64) > lynx.SCRATCH_BYTES
    with pytest.raises(lynx.LynxError, match="LYNX_ERR_SCRATCH"):
        lynx.linear_sparse_lora_noalloc(X, W, LA, LB)
