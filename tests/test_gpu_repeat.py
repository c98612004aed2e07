"""Repeated calls give the same bytes, and the debug mode changes nothing but
the wait.

- Determinism at full size: the sparse + LoRA layer and the dense layer at
  MLP-up (256-wide tiles, three rounds of the persistent GEMM) and MLP-down
  (192-wide tiles, K = 12288). Each gets three calls, each into freshly
  poisoned outputs and workspaces, and Y must be the same bytes every time.
  Nothing on the path uses atomics or an order-dependent reduction, so a race
  in the LDS rings or in the cross-wave reductions would show here.
- Debug mode (LYNX_DEBUG=1): every entry point returns LYNX_OK and writes the
  same bytes as without it. A graph captured in debug mode, where the wait is
  skipped on the capturing stream, replays to the same bytes.
"""
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from tests.gpu_util import dev, say
from workloads import make_config, make_layer

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16).clone() if t.dtype == torch.bfloat16 else t.clone()


@pytest.mark.parametrize("config", ["mlp_up", "mlp_down"])
def test_full_size_layers_are_deterministic(config):
    (L,) = make_config(config, seed=3)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    first = None
    for i in range(3):
        say(f"determinism {config} M={L.M} K={L.K} N={L.N} call {i}")
        got = (bits(gu.sparse_lora(X, W, LA, LB)), bits(gu.dense(X, W)))
        torch.cuda.synchronize()
        assert not torch.any(got[0] == gu.NAN_BF16_BITS), f"{config}: Y not fully written"
        if first is None:
            first = got
        else:
            assert torch.equal(got[0], first[0]), f"{config}: sparse layer, call {i} differs"
            assert torch.equal(got[1], first[1]), f"{config}: dense layer, call {i} differs"


def run_every_entry_point(X, W, LA, LB):
    M, N = X.shape[0], W.shape[0]
    out = {"sparse_lora": gu.sparse_lora(X, W, LA, LB),
           "noalloc": gu.sparse_lora_noalloc(X, W, LA, LB),
           "dense": gu.dense(X, W)}
    values, meta, scale, T = gu.sparsify(X, LB)
    out.update(values=values, meta=meta, scale=scale, T=T)
    out["packed"] = gu.packed(values, meta, scale, T, W, LA)
    layers = [dict(X=X, W=W, LA=LA, LB=LB, Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")),
              dict(X=X, W=W, Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), dense=True)]
    gu.sequence(layers)
    out["sequence_sparse"], out["sequence_dense"] = layers[0]["Y"], layers[1]["Y"]
    torch.cuda.synchronize()
    return {k: bits(v) for k, v in out.items()}


def test_debug_mode_writes_the_same_bytes_and_captures(monkeypatch):
    M, K, N, R = 1024, 512, 1024, 64      # the tiled kernels
    L = make_layer(M, K, N, "heavy", seed=11, R=R)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    monkeypatch.delenv("LYNX_DEBUG", raising=False)
    say("debug mode: reference calls")
    ref = run_every_entry_point(X, W, LA, LB)
    monkeypatch.setenv("LYNX_DEBUG", "1")
    say("debug mode: LYNX_DEBUG=1 calls")
    got = run_every_entry_point(X, W, LA, LB)
    for k in ref:
        assert torch.equal(got[k], ref[k]), f"debug mode changed {k}"

    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say("debug mode: graph capture of the no-allocation layer")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lynx.linear_sparse_lora_noalloc(X, W, LA, LB, Y=Y)
    for i in range(3):
        Y.view(torch.int16).fill_(gu.NAN_BF16_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(Y), ref["noalloc"]), f"debug-mode graph replay {i} differs"
