"""Pin the gfx950 matrix-instruction operand layouts on the device.

One instruction per wave runs on random small-integer operands (every sum is
exact in fp32) and random valid sparse-index words; the result must equal
the dense product under the documented lane maps.  This pins what the packed
format (include/lynx.h) and the GEMM kernels assume:

  v_smfmac_f32_16x16x64_bf16, lane l, r = l % 16, q = l / 16:
    A: row r; its 8 values are the kept entries of dense channels
       [16q, 16q+16) = 4 groups; value 2g+s of group g sits at channel
       16q + 4g + ((idx >> (4g + 2s)) & 3), idx = the 16-bit word picked by abid;
    B: column r; element e holds channel 8q + (e % 8) + 32 (e / 8), i.e. the
       two 8-channel chunks q and 4 + q of the 64-channel step;
    D: column r, rows 4q .. 4q+3.
  v_smfmac_f32_32x32x32_bf16: A as above with r = l % 32, q = l / 32 over a
    32-channel step; B element e holds channel 8q + (e % 8) + 16 (e / 8);
    32x32 accumulator map row = 8 (e / 4) + 4 q + e % 4, column r.
  (Only the relative A/B channel map is observable; this is one consistent
  description of it, found by testing candidate maps on the raw results.)
  v_mfma_f32_16x16x32_bf16: A row r, B column r, channels 8q .. 8q+7.
  v_mfma_f32_32x32x16_bf16: A row l % 32, B column l % 32, channels 8 (l/32) + e.
"""
import numpy as np
import pytest
import torch

from activation_sparse_gemm_amd import _abi
from tests.gpu_util import dump_dir, say

pytestmark = pytest.mark.gpu

PAIRS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


def bf16_small_ints(rng, shape):
    v = rng.integers(-4, 5, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16), v


def random_index_words(rng, n):
    words = np.zeros(n, dtype=np.uint32)
    for half in range(2):
        for g in range(4):
            p = rng.integers(0, 6, size=n)
            code = np.array([PAIRS[i][0] | (PAIRS[i][1] << 2) for i in p], dtype=np.uint32)
            words |= code << (16 * half + 4 * g)
    return words


def expand_sparse(a, idx, abid, nrow, kdense, lane_row, lane_kb):
    A = np.zeros((nrow, kdense))
    for l in range(64):
        w = (int(idx[l]) >> (16 * abid)) & 0xFFFF
        for e in range(8):
            g, s = divmod(e, 2)
            pos = (w >> (4 * g + 2 * s)) & 3
            A[lane_row(l), lane_kb(l) + 4 * g + pos] = a[l, e]
    return A


def acc_16(D):
    d = np.zeros((64, 4))
    for l in range(64):
        for e in range(4):
            d[l, e] = D[4 * (l // 16) + e, l % 16]
    return d


def acc_32(D):
    d = np.zeros((64, 16))
    for l in range(64):
        for e in range(16):
            d[l, e] = D[8 * (e // 4) + 4 * (l // 32) + e % 4, l % 32]
    return d


def run(which, abid, a_bits, b_bits, idx, dshape):
    a = torch.from_numpy(a_bits.view(np.int16)).cuda()
    b = torch.from_numpy(b_bits.view(np.int16)).cuda()
    ix = torch.from_numpy(idx.view(np.int32)).cuda()
    d = torch.zeros(dshape, dtype=torch.float32, device="cuda")
    say(f"probe which={which} abid={abid}")
    _abi.probe_mfma(which, abid, a, b, ix, d)
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("abid", [0, 1])
def test_smfmac_16x16x64_layout(abid):
    rng = np.random.default_rng(100 + abid)
    a_bits, a = bf16_small_ints(rng, (64, 8))
    b_bits, b = bf16_small_ints(rng, (64, 16))
    idx = random_index_words(rng, 64)
    d = run(0, abid, a_bits, b_bits, idx, (64, 4))
    if dump_dir():
        np.savez(f"{dump_dir()}/probe_s16_{abid}.npz", a=a, b=b, idx=idx, d=d)
    A = expand_sparse(a, idx, abid, 16, 64, lambda l: l % 16, lambda l: 16 * (l // 16))
    B = np.zeros((64, 16))
    for l in range(64):
        for e in range(16):
            B[8 * (l // 16) + (e % 8) + 32 * (e // 8), l % 16] = b[l, e]
    np.testing.assert_array_equal(d, acc_16(A @ B))


@pytest.mark.parametrize("abid", [0, 1])
def test_smfmac_32x32x32_layout(abid):
    rng = np.random.default_rng(200 + abid)
    a_bits, a = bf16_small_ints(rng, (64, 8))
    b_bits, b = bf16_small_ints(rng, (64, 16))
    idx = random_index_words(rng, 64)
    d = run(1, abid, a_bits, b_bits, idx, (64, 16))
    if dump_dir():
        np.savez(f"{dump_dir()}/probe_s32_{abid}.npz", a=a, b=b, idx=idx, d=d)
    A = expand_sparse(a, idx, abid, 32, 32, lambda l: l % 32, lambda l: 16 * (l // 32))
    B = np.zeros((32, 32))
    for l in range(64):
        for e in range(16):
            B[8 * (l // 32) + (e % 8) + 16 * (e // 8), l % 32] = b[l, e]
    np.testing.assert_array_equal(d, acc_32(A @ B))


def test_mfma_16x16x32_layout():
    rng = np.random.default_rng(300)
    a_bits, a = bf16_small_ints(rng, (64, 8))
    b_bits, b = bf16_small_ints(rng, (64, 8))
    d = run(2, 0, a_bits, b_bits, np.zeros(64, np.uint32), (64, 4))
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for l in range(64):
        A[l % 16, 8 * (l // 16): 8 * (l // 16) + 8] = a[l]
        B[8 * (l // 16): 8 * (l // 16) + 8, l % 16] = b[l]
    np.testing.assert_array_equal(d, acc_16(A @ B))


def test_mfma_32x32x16_layout():
    rng = np.random.default_rng(400)
    a_bits, a = bf16_small_ints(rng, (64, 8))
    b_bits, b = bf16_small_ints(rng, (64, 8))
    d = run(3, 0, a_bits, b_bits, np.zeros(64, np.uint32), (64, 16))
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for l in range(64):
        A[l % 32, 8 * (l // 32): 8 * (l // 32) + 8] = a[l]
        B[8 * (l // 32): 8 * (l // 32) + 8, l % 32] = b[l]
    np.testing.assert_array_equal(d, acc_32(A @ B))


def test_matrix_instruction_issue_rates():
    """The peaks the roofline uses: the 32x32 bf16 forms issue once per 32
    cycles per SIMD, the 2:4 one doing twice the dense one's work, and the
    16x16x64 2:4 form about once per 16; the shader clock under that load
    lies within the chip's range."""
    import numpy as np

    from activation_sparse_gemm_amd import _abi
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    expect = {0: (15.5, 18.5), 1: (31.5, 33.5), 3: (31.5, 33.5)}
    for which, (lo, hi) in expect.items():
        say(f"issue rate of {_abi.PROBE_NAMES[which]}")
        r = _abi.probe_mfma_rate(which, 1024, cus)
        st = r["stamps"].astype(np.float64)
        assert np.all(st[:, 0] > 0) and np.all(st[:, 1] > 0)
        cpi = float(np.median(st[:, 0])) / (16 * 1024)
        mhz = float(np.median(100.0 * st[:, 0] / st[:, 1]))
        say(f"  {cpi:.2f} cycles per instruction at {mhz:.0f} MHz")
        assert lo <= cpi <= hi, cpi
        assert 800.0 <= mhz <= 2500.0, mhz
    assert _abi.PROBE_FLOPS[1] == 2 * _abi.PROBE_FLOPS[3]
