"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in the CPU oracle (monkeypatching a function)
and checks that at least one pin of test_oracle_pins fails.  Nothing here
touches a GPU.
"""
import numpy as np
import pytest

from oracle import lynx_oracle as orc
from tests import test_oracle_pins as pins

PIN_TESTS = [
    lambda: pins.test_select_exhaustive_tie_patterns(),
    lambda: pins.test_golden_worked_example(),
    lambda: pins.test_norm_preserved_and_scale_bounds("heavy"),
    lambda: pins.test_zero_row(),
    lambda: pins.test_two_sparse_input_without_lora_is_dense_gemm(),
    lambda: pins.test_zero_weight_leaves_lora_of_dense_x(),
    lambda: pins.test_all_plus_minus_one_closed_form(),
    lambda: pins.test_tiny_layer_brute_force(4, 32, 5, 3, 0),
    lambda: pins.test_tiny_layer_brute_force(3, 16, 8, 2, 1),
    lambda: pins.test_packed_path_with_lora_brute_force(),
]


def _some_pin_fails():
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _ties_to_higher_index(X_bits):
    x = orc.decode_bf16(X_bits)
    M, K = x.shape
    mag = np.abs(x).reshape(M, K // 4, 4)[..., ::-1]
    order = 3 - np.argsort(-mag, axis=-1, kind="stable")[..., :2]
    return np.sort(order, axis=-1).astype(np.int64)


def _inverted_scale(x, mask):
    s = orc_norm_scale_orig(x, mask)
    return 1.0 / s


def _scale_without_sqrt(x, mask):
    s = orc_norm_scale_orig(x, mask)
    return s * s


def _meta_swapped_nibbles(idx):
    code = (idx[..., 1] | (idx[..., 0] << 2)).astype(np.uint8)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)


def _meta_swapped_groups(idx):
    code = (idx[..., 0] | (idx[..., 1] << 2)).astype(np.uint8)
    return (code[:, 1::2] | (code[:, 0::2] << 4)).astype(np.uint8)


def _layer_lora_on_sparse_x(X_bits, W_bits, LA_bits=None, LB_bits=None):
    x = orc.decode_bf16(X_bits)
    mask = orc.keep_mask(orc.select_top2_of_4(X_bits))
    s = orc.norm_scale(x, mask)
    xt = np.where(mask, x, 0.0)
    Y = s[:, None] * (xt @ orc.decode_bf16(W_bits).T)
    if LA_bits is not None and LB_bits is not None:
        Y = Y + (xt @ orc.decode_bf16(LB_bits).T) @ orc.decode_bf16(LA_bits).T
    return Y


def _layer_scaled_lora(X_bits, W_bits, LA_bits=None, LB_bits=None):
    x = orc.decode_bf16(X_bits)
    mask = orc.keep_mask(orc.select_top2_of_4(X_bits))
    s = orc.norm_scale(x, mask)
    Y = orc_linear_orig(X_bits, W_bits, LA_bits, LB_bits)
    if LA_bits is not None and LB_bits is not None:
        Yr = (x @ orc.decode_bf16(LB_bits).T) @ orc.decode_bf16(LA_bits).T
        Y = Y + (s[:, None] - 1.0) * Yr
    return Y


def _layer_dropped_lora(X_bits, W_bits, LA_bits=None, LB_bits=None):
    return orc_linear_orig(X_bits, W_bits, None, None)


def _layer_negated_lora(X_bits, W_bits, LA_bits=None, LB_bits=None):
    Y = orc_linear_orig(X_bits, W_bits, None, None)
    if LA_bits is not None and LB_bits is not None:
        x = orc.decode_bf16(X_bits)
        Y = Y - (x @ orc.decode_bf16(LB_bits).T) @ orc.decode_bf16(LA_bits).T
    return Y


def _layer_lora_la_lb_swapped_roles(X_bits, W_bits, LA_bits=None, LB_bits=None):
    # uses row index of LA for the rank: wrong orientation of the up-projection
    Y = orc_linear_orig(X_bits, W_bits, None, None)
    if LA_bits is not None and LB_bits is not None:
        x = orc.decode_bf16(X_bits)
        T = x @ orc.decode_bf16(LB_bits).T
        LA = orc.decode_bf16(LA_bits)
        Y = Y + T @ np.flip(LA, axis=0).T
    return Y


def _packed_dropped_lora(values, meta, scale, T_bits, W_bits, LA_bits, K):
    return orc_packed_orig(values, meta, scale, None, W_bits, None, K)


def _packed_lora_scaled_by_s(values, meta, scale, T_bits, W_bits, LA_bits, K):
    # s applied after the LoRA term: s (X~ W^T + T LA^T)
    Y = orc_packed_orig(values, meta, scale, T_bits, W_bits, LA_bits, K)
    if T_bits is not None and LA_bits is not None:
        Yr = orc.decode_bf16(T_bits) @ orc.decode_bf16(LA_bits).T
        Y = Y + (np.asarray(scale, dtype=np.float64)[:, None] - 1.0) * Yr
    return Y


def _packed_lora_transposed_la(values, meta, scale, T_bits, W_bits, LA_bits, K):
    Y = orc_packed_orig(values, meta, scale, None, W_bits, None, K)
    if T_bits is not None and LA_bits is not None:
        LA = orc.decode_bf16(LA_bits)
        Y = Y + orc.decode_bf16(T_bits) @ np.flip(LA, axis=1).T
    return Y


orc_norm_scale_orig = orc.norm_scale
orc_linear_orig = orc.linear_sparse_lora
orc_packed_orig = orc.linear_from_packed

MUTATIONS = {
    "ties_to_higher_index": ("select_top2_of_4", _ties_to_higher_index),
    "inverted_scale": ("norm_scale", _inverted_scale),
    "scale_without_sqrt": ("norm_scale", _scale_without_sqrt),
    "meta_swapped_nibbles": ("pack_meta", _meta_swapped_nibbles),
    "meta_swapped_groups": ("pack_meta", _meta_swapped_groups),
    "lora_on_sparse_x": ("linear_sparse_lora", _layer_lora_on_sparse_x),
    "scaled_lora": ("linear_sparse_lora", _layer_scaled_lora),
    "dropped_lora": ("linear_sparse_lora", _layer_dropped_lora),
    "negated_lora": ("linear_sparse_lora", _layer_negated_lora),
    "misoriented_lora_up": ("linear_sparse_lora", _layer_lora_la_lb_swapped_roles),
    "packed_dropped_lora": ("linear_from_packed", _packed_dropped_lora),
    "packed_lora_scaled_by_s": ("linear_from_packed", _packed_lora_scaled_by_s),
    "packed_lora_rank_order_flipped": ("linear_from_packed", _packed_lora_transposed_la),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert _some_pin_fails(), f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_all_pins():
    assert not _some_pin_fails()
