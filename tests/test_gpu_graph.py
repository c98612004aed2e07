"""The layer under HIP graph capture: the no-allocation entry point (for the
callers include/lynx.h names, such as code under graph capture), the
workspace entry point and the block driver, captured once with
torch.cuda.graph and replayed three times.

Before each replay the outputs are refilled with a NaN pattern and other
eager work runs on the GPU (a dense layer over other buffers); every replay's
Y must equal the eager call's bit for bit.  No hipMemsetAsync is recorded:
the library's calls launch only its own kernels.
"""
import numpy as np
import pytest
import torch

import activation_sparse_gemm_amd as lynx
import tests.gpu_util as gu
from tests.gpu_util import dev, say
from workloads import make_layer

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16).clone()


def replay_and_check(g, outputs, refs, label):
    other = make_layer(512, 512, 768, "heavy", seed=99, R=16)
    Xo, Wo = dev(other.X), dev(other.W)
    for i in range(3):
        for Y in outputs:
            Y.view(torch.int16).fill_(gu.NAN_BF16_BITS)
        lynx.linear_dense(Xo, Wo)              # eager work between the replays
        torch.cuda.synchronize()
        say(f"graph replay {i}: {label}")
        g.replay()
        torch.cuda.synchronize()
        for Y, ref in zip(outputs, refs):
            assert torch.equal(Y.view(torch.int16), ref), f"{label}: replay {i} differs from eager"


@pytest.mark.parametrize("M,K,N,R", [(1024, 512, 1024, 64), (256, 512, 512, 64)])
def test_noalloc_layer_replays_in_a_graph(M, K, N, R):
    L = make_layer(M, K, N, "heavy", seed=M + N, R=R)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    say(f"graph: noalloc eager M={M} K={K} N={N}")
    lynx.linear_sparse_lora_noalloc(X, W, LA, LB, Y=Y)
    torch.cuda.synchronize()
    ref = bits(Y)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lynx.linear_sparse_lora_noalloc(X, W, LA, LB, Y=Y)
    replay_and_check(g, [Y], [ref], f"noalloc {M}x{K}->{N}")


def test_workspace_layer_replays_in_a_graph():
    M, K, N, R = 256, 512, 512, 64        # the 64 x 64 kernels
    L = make_layer(M, K, N, "heavy", seed=5, R=R)
    X, W, LA, LB = dev(L.X), dev(L.W), dev(L.LA), dev(L.LB)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((lynx.workspace_bytes(M, K, R),), dtype=torch.uint8, device="cuda")
    say("graph: workspace layer eager")
    lynx.linear_sparse_lora(X, W, LA, LB, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    ref = bits(Y)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lynx.linear_sparse_lora(X, W, LA, LB, Y=Y, workspace=ws)
    replay_and_check(g, [Y], [ref], "workspace layer")


def test_block_driver_replays_in_a_graph():
    specs = [(1024, 512, 1536, False), (1024, 1536, 512, True), (1024, 512, 1024, False)]
    layers = []
    for i, (M, K, N, skipped) in enumerate(specs):
        L = make_layer(M, K, N, "heavy", seed=20 + i, R=32)
        layers.append(dict(X=dev(L.X), W=dev(L.W), LA=dev(L.LA), LB=dev(L.LB),
                           Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                           dense=skipped))
    ws = torch.empty((max(lynx.sequence_workspace_bytes(layers), 1),), dtype=torch.uint8,
                     device="cuda")
    say("graph: block driver eager")
    lynx.linear_sequence(layers, workspace=ws)
    torch.cuda.synchronize()
    refs = [bits(d["Y"]) for d in layers]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lynx.linear_sequence(layers, workspace=ws)
    replay_and_check(g, [d["Y"] for d in layers], refs, "block driver")
