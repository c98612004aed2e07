"""The sparse GEMM's schedule (lynx_probe_sparse_plan): whole tiles and
stream-K tiles, checked on the host for many shapes and compute-unit counts.

The stream-K split, as include/lynx_probe.h states it: range rho of the
grid's P ranges takes the stage pairs floor(rho * pairs / P) ..
floor((rho + 1) * pairs / P) - 1 of the stream-K tiles (tile t holds pairs
t * K/128 .. (t + 1) * K/128 - 1); workgroup w runs range
(w % 8) * P/8 + w / 8 when P % 8 == 0 (else range w), then its whole tiles
w, w + P, ... below the whole-tile count.  A segment that holds a tile's
first stage owns the tile; any other segment is a partial sum that its
workgroup hands to the owner.  From that definition this test checks, for
every planned shape:
  * every stage of every tile is computed exactly once;
  * each stream-K tile has exactly one segment starting at its first stage;
  * a partial segment is always the first unit of its workgroup (so no
    segment that an owner waits for waits itself: the waits cannot cycle)
    and each workgroup has at most one (its partial-sum slot is unique);
  * no tile has more than two partial sums (what the kernel's owners add);
  * segments are whole stage pairs (>= 2 stages, what the kernel's ring needs);
  * lynx_workspace_bytes adds exactly the plan's partial-sum slots and flags.
No GPU is used (the plan is host code; with no device it assumes 256 CUs).
"""
import itertools

import pytest

from activation_sparse_gemm_amd import _abi

SHAPES = [
    (4096, 9216, 3072), (4096, 12288, 3072), (4096, 3072, 12288),           # QKV, MLP-up, -down
    (9216, 9216, 3072), (9216, 3072, 3072), (9216, 12288, 3072), (9216, 3072, 12288),  # block
    (4096, 4352, 512), (4000, 4300, 512), (1024, 1024, 192), (1000, 1100, 320),
    (8192, 8192, 8192), (300, 20000, 1024), (20000, 300, 2048), (2048, 2304, 448),
    (4096, 4096, 128), (1536, 5000, 6400), (5120, 1280, 64),
]
CUS = [256, 80, 32, 304, 8, 300]


def tiles_of(M, N, width):
    return ((M + 255) // 256) * ((N + width - 1) // width)


def simulate(plan, K):
    """Units of every workgroup, from the documented split."""
    P, nk = plan["grid"], K // 64
    half = nk // 2
    units = {w: [] for w in range(P)}
    if plan["sk_tiles"]:
        pairs = plan["pairs"]
        assert pairs == plan["sk_tiles"] * half and pairs >= P
        for w in range(P):
            rho = (w % 8) * (P // 8) + w // 8 if P % 8 == 0 else w
            s0, s1 = 2 * (rho * pairs // P), 2 * ((rho + 1) * pairs // P)
            s = s0
            while s < s1:
                t = s // nk
                e = min(s1, (t + 1) * nk)
                units[w].append(("sk", plan["dp_tiles"] + t, s - t * nk, e - s, rho))
                s = e
    for w in range(P):
        b = w
        while b < plan["dp_tiles"]:
            units[w].append(("whole", b, 0, nk, None))
            b += P
    return units


def check_plan(M, N, K, cus, with_sk):
    plan = _abi.sparse_plan(M, N, K, with_sk, cus)
    tiles_total = None
    if not plan["tiled"]:
        assert (M + 255) // 256 * ((N + 255) // 256) < 16 or K < 128
        return plan
    assert plan["width"] in (192, 256)
    tiles_total = tiles_of(M, N, plan["width"])
    assert plan["dp_tiles"] + plan["sk_tiles"] == tiles_total
    nk = K // 64
    if plan["sk_tiles"] == 0:
        assert plan["grid"] == min(tiles_total, cus) and plan["partial_bytes"] == 0
        assert plan["flag_bytes"] == 0
        return plan
    assert with_sk and nk % 2 == 0 and plan["grid"] == cus
    assert plan["dp_tiles"] % cus == 0
    assert plan["partial_bytes"] == cus * 4 * 64 * 64 * (plan["width"] // 64) * 4
    assert plan["flag_bytes"] == (4 * plan["sk_tiles"] + 255) // 256 * 256
    units = simulate(plan, K)
    cover = {}
    first_stage = {}
    partials = {}
    for w, us in units.items():
        for i, (kind, bid, kb, ln, rho) in enumerate(us):
            assert ln >= 2 and ln % 2 == 0 and kb % 2 == 0
            for k in range(kb, kb + ln):
                key = (bid, k)
                assert key not in cover, f"stage {key} computed twice"
                cover[key] = w
            if kind == "sk":
                if kb == 0:
                    assert bid not in first_stage
                    first_stage[bid] = rho
                else:
                    assert i == 0, "a partial sum that is not its workgroup's first unit"
                    partials.setdefault(bid, []).append(rho)
    assert len(cover) == tiles_total * nk
    assert sum(len(v) for v in partials.values()) <= cus
    for t in range(plan["dp_tiles"], tiles_total):
        assert t in first_stage
        got = sorted(partials.get(t, []))
        assert len(got) <= 2
        # the owner waits for ranges rho + 1 .. last: exactly these partials
        assert got == list(range(first_stage[t] + 1, first_stage[t] + 1 + len(got)))
    return plan


@pytest.mark.parametrize("cus", CUS)
def test_schedule_covers_every_stage_once(cus):
    for (M, N, K), with_sk in itertools.product(SHAPES, (True, False)):
        plan = check_plan(M, N, K, cus, with_sk)
        if not with_sk:
            assert plan["sk_tiles"] == 0


def test_workspace_adds_the_plan_stream_k_region():
    """Without a GPU the plan assumes 256 compute units, as the workspace query does."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("on a GPU the workspace follows the device's compute-unit count")
    for (M, N, K) in SHAPES:
        R = 64
        plan = _abi.sparse_plan(M, N, K, True, 256)
        Mp = (M + 15) // 16 * 16
        r256 = lambda x: (x + 255) // 256 * 256
        base = r256(Mp * K) + r256(Mp * K // 8) + r256(4 * M) + r256(2 * M * R)
        assert _abi.workspace_bytes(M, N, K, R) == base + plan["partial_bytes"] + plan["flag_bytes"]


def test_workload_schedules():
    """The schedules the cost model picks for the DiT workloads on 256 CUs."""
    want = {
        (4096, 12288, 3072): (256, 0),      # MLP-up: three full rounds
        (4096, 9216, 3072): (256, 320),     # QKV: one round whole, 1.25 stream-K
        (4096, 3072, 12288): (256, 192),    # MLP-down: 0.75 of a round, all stream-K
        (9216, 3072, 3072): (256, 432),     # block attention-out: 1.69 rounds
        (9216, 3072, 12288): (256, 432),    # block MLP-down
        (9216, 9216, 3072): (256, 272),     # block QKV: 5.06 rounds
        (9216, 12288, 3072): (256, 0),      # block MLP-up: 6.75 rounds, whole tiles
    }
    for (M, N, K), (width, sk) in want.items():
        plan = _abi.sparse_plan(M, N, K, True, 256)
        assert (plan["width"], plan["sk_tiles"]) == (width, sk), (M, N, K, plan)


def test_plan_validation():
    out = (_abi.ctypes.c_int64 * 8)()
    L = _abi.lib()
    assert L.lynx_probe_sparse_plan(16, 16, 96, 1, 256, out) == 2     # K % 64
    assert L.lynx_probe_sparse_plan(16, 16, 128, 1, 0, out) == 2      # cus
    assert L.lynx_probe_sparse_plan(0, 16, 128, 1, 256, out) == 2     # empty
    assert L.lynx_probe_sparse_plan(16, 16, 128, 1, 256, None) == 1
