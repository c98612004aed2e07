"""Calls on two streams at once: the library keeps no per-call state, so two
layers running concurrently on separate streams, each with its own inputs,
outputs and workspace, must give the same bytes as the same calls run one
after the other.

Both streams have the default priority. The persistent GEMMs take one
workgroup per compute unit and never wait on another workgroup, so two of them
in flight only share the compute units.
"""
import pytest
import torch

import activation_sparse_gemm_amd as lynx
from tests.gpu_util import dev, say
from workloads import make_layer

pytestmark = pytest.mark.gpu


def layer_inputs(M, K, N, R, seed):
    L = make_layer(M, K, N, "heavy", seed=seed, R=R)
    return dict(X=dev(L.X), W=dev(L.W), LA=dev(L.LA), LB=dev(L.LB),
                ws=torch.empty(lynx.workspace_bytes(M, K, R), dtype=torch.uint8, device="cuda"),
                Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                Yd=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))


def run(d):
    lynx.linear_sparse_lora(d["X"], d["W"], d["LA"], d["LB"], Y=d["Y"], workspace=d["ws"])
    lynx.linear_dense(d["X"], d["W"], Y=d["Yd"])


def test_two_streams_give_the_sequential_bytes():
    a = layer_inputs(2048, 1024, 3072, 64, seed=31)     # tiled kernels
    b = layer_inputs(1536, 2048, 2048, 32, seed=32)
    say("streams: sequential reference")
    run(a)
    run(b)
    torch.cuda.synchronize()
    ref = [t.view(torch.int16).clone() for t in (a["Y"], a["Yd"], b["Y"], b["Yd"])]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for d in (a, b):
            d["Y"].view(torch.int16).fill_(0x7FC0)
            d["Yd"].view(torch.int16).fill_(0x7FC0)
        torch.cuda.synchronize()
        say(f"streams: concurrent round {rep}")
        for _ in range(4):
            with torch.cuda.stream(s1):
                run(a)
            with torch.cuda.stream(s2):
                run(b)
        torch.cuda.synchronize()
        got = [t.view(torch.int16) for t in (a["Y"], a["Yd"], b["Y"], b["Yd"])]
        for name, g, r in zip(("A sparse", "A dense", "B sparse", "B dense"), got, ref):
            assert torch.equal(g, r), f"round {rep}: {name} differs from the sequential call"
