"""lynx_linear_sequence (the block driver with selective layer skipping)
against the CPU oracle's linear_sequence.

Bar: as for single layers, per-row relative Frobenius error of every layer's
Y <= 5e-3, zero reference rows exactly zero, no non-finite output; and each
layer's output bit-identical to the same layer run through its own entry
point (the sequence only orders the same kernels).
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from oracle import lynx_oracle as orc
from tests.gpu_util import ROW_REL_TOL, dev, host_f64, report, sample_rows, say
from workloads import BLOCK_LAYER_NAMES, make_config, make_layer

pytestmark = pytest.mark.gpu


def check(Yg, Yref, label):
    Yg = host_f64(Yg)
    rep = report(label, Yg, Yref)
    zero = np.linalg.norm(Yref, axis=1) == 0
    assert np.all(Yg[zero] == 0), f"{label}: zero rows"
    assert rep["nonfinite"] == 0 and rep["max_row_rel"] <= ROW_REL_TOL, label


def as_device(L, skipped):
    return dict(X=dev(L.X), W=dev(L.W), LA=dev(L.LA), LB=dev(L.LB),
                Y=torch.empty((L.M, L.N), dtype=torch.bfloat16, device="cuda"), dense=skipped)


def test_mixed_small_sequence():
    # both GEMM kernel families, ragged shapes, and an empty layer
    specs = [(300, 1152, 257, False), (513, 384, 520, True), (1000, 640, 1100, False),
             (1024, 128, 1024, True), (0, 256, 64, False), (37, 2048, 300, False)]
    Ls = [make_layer(M, K, N, "heavy", seed=11 + i) for i, (M, K, N, _) in enumerate(specs)]
    layers = [as_device(L, sk) for L, (_, _, _, sk) in zip(Ls, specs)]
    say("sequence of 6 layers, two skipped")
    gu.sequence(layers)
    torch.cuda.synchronize()
    refs = orc.linear_sequence([(L.X, L.W, L.LA, L.LB, sk) for L, (_, _, _, sk) in zip(Ls, specs)])
    for i, (d, ref) in enumerate(zip(layers, refs)):
        if d["Y"].numel():
            check(d["Y"], ref, f"layer {i} ({'dense' if specs[i][3] else 'sparse'})")
    # the same kernels as the single-layer entry points, bit for bit
    for d in layers:
        if not d["Y"].numel():
            continue
        if d["dense"]:
            Y1 = gu.dense(d["X"], d["W"])
        else:
            Y1 = gu.sparse_lora(d["X"], d["W"], d["LA"], d["LB"])
        torch.cuda.synchronize()
        assert torch.equal(Y1.view(torch.int16), d["Y"].view(torch.int16))


@pytest.mark.parametrize("skip", [(), ("attn_out", "mlp_up")])
def test_block_sequence_sampled_rows(skip):
    Ls = make_config("block")
    flags = [name in skip for name in BLOCK_LAYER_NAMES]
    layers = [as_device(L, sk) for L, sk in zip(Ls, flags)]
    say(f"block sequence, skipped: {skip or 'none'}")
    gu.sequence(layers)
    torch.cuda.synchronize()
    for i, (L, d, sk) in enumerate(zip(Ls, layers, flags)):
        rows = sample_rows(L.M, n=16, seed=i)
        Yh = host_f64(d["Y"])[rows]
        (ref,) = orc.linear_sequence([(L.X[rows], L.W, L.LA, L.LB, sk)])
        check(torch.from_numpy(Yh), ref, f"block {BLOCK_LAYER_NAMES[i]} ({'dense' if sk else 'sparse'})")
        del d["Y"]
