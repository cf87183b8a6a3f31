"""Test the tests: plant plausible mistakes in the oracle (on the CPU) and require a pin to fail.

Each mutation replaces one oracle function with a subtly wrong variant for the
duration of one test; the listed pin tests must then fail. This shows the pins
are sensitive to the mistakes they are meant to catch, rather than merely
passing.
"""

import os

import numpy as np
import pytest

import tests.test_oracle_pins as pins
from oracle import dsa_oracle as O


def _no_relu(q, w, keys):
    return w @ (q @ keys.T)


def _reversed_head_weights(q, w, keys):
    return w[::-1] @ np.maximum(q @ keys.T, 0.0)


def _relu_after_sum(q, w, keys):
    return np.maximum(w @ (q @ keys.T), 0.0)


_orig_scores = O.indexer_scores


def _causal_off_by_one(host, rows=None):
    out = _orig_scores(host, rows)
    return {r: s[:-1] for r, s in out.items()}


def _reversed_ties(scores, k):
    s = np.asarray(scores, dtype=np.float64)
    n = min(k, s.shape[0])
    order = np.lexsort((-np.arange(len(s)), -s))[:n]  # ties toward higher positions
    out = np.full(k, -1, dtype=np.int32)
    out[:n] = np.sort(order)
    return out


def _unscaled_mla(q, rows, scale, d_latent):
    return _orig_mla_row(q, rows, 1.0, d_latent)


_orig_mla_row = O.sparse_mla_row


def _value_with_rope(q, rows, scale, d_latent):
    o, lse = _orig_mla_row(q, rows, scale, rows.shape[1])
    return o[:, -d_latent:], lse


def _no_block_table(block_table, b, positions, page_size):
    positions = np.asarray(positions, dtype=np.int64)
    return positions // page_size, positions % page_size


def _wrong_sequence_table(block_table, b, positions, page_size):
    positions = np.asarray(positions, dtype=np.int64)
    return block_table[0, positions // page_size].astype(np.int64), positions % page_size


_orig_keys = O.indexer_keys


def _fp8_scale_ignored(host, b, n):
    h = dict(host)
    if h["idx_k_dtype"] == "fp8":
        h["k_scale"] = np.ones_like(np.asarray(h["k_scale"]))
    return _orig_keys(h, b, n)


def _e4m3_fnuz(codes):
    # the other common e4m3 flavour: bias 8, 0x80 is NaN
    tab = O.e4m3fn_table() / 2.0
    tab[0x80] = np.nan
    return tab[np.asarray(codes, dtype=np.uint8)]


def _e4m3_ties_away(x):
    # round half away from zero instead of to the even code
    x = np.asarray(x, dtype=np.float32)
    tab = O.e4m3fn_table()[:0x7F]
    flat = x.reshape(-1).astype(np.float64)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        d = np.abs(tab - abs(v))
        out[i] = int(np.flatnonzero(d == d.min())[-1]) | (0x80 if np.signbit(v) else 0)
    return out.reshape(x.shape)


def _e4m3_truncate(x):
    # round toward zero
    x = np.asarray(x, dtype=np.float32)
    tab = O.e4m3fn_table()[:0x7F]
    flat = x.reshape(-1).astype(np.float64)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        out[i] = int(np.flatnonzero(tab <= abs(v))[-1]) | (0x80 if np.signbit(v) else 0)
    return out.reshape(x.shape)


_orig_quant = O.quantize_key_e4m3


def _scale_by_255(k):
    # the scale of an int8-style format instead of e4m3's 448
    k = np.asarray(k, dtype=np.float32)
    sigma = np.float32(np.max(np.abs(k))) / np.float32(255.0)
    return O.e4m3fn_encode(np.clip(k / sigma, -448, 448).astype(np.float32)), sigma


def _page_sum(token_scores, page_size):
    # rank a page by the sum of its scores instead of the maximum
    s = np.asarray(token_scores, dtype=np.float64)
    n = (len(s) + page_size - 1) // page_size
    return np.array([s[p * page_size:(p + 1) * page_size].sum() for p in range(n)])


def _expand_past_t(pages, page_size, t):
    # read whole pages, also the positions past t
    out = np.full(len(pages) * page_size, -1, dtype=np.int32)
    for i, p in enumerate(pages):
        if p >= 0:
            out[i * page_size:(i + 1) * page_size] = np.arange(p * page_size, (p + 1) * page_size)
    return out


MUTATIONS = [
    ("page_scores_row", _page_sum, ["test_page_budget_worked_example",
                                    "test_page_budget_brute_force_with_masked_future"]),
    ("expand_pages", _expand_past_t, ["test_page_budget_brute_force_with_masked_future"]),
    ("e4m3fn_encode", _e4m3_ties_away, ["test_e4m3_encode_round_trip_and_ties_to_even",
                                        "test_e4m3_encode_matches_torch_cast"]),
    ("e4m3fn_encode", _e4m3_truncate, ["test_e4m3_encode_round_trip_and_ties_to_even",
                                       "test_e4m3_encode_matches_torch_cast"]),
    ("quantize_key_e4m3", _scale_by_255, ["test_quantize_key_scale_and_error_bound",
                                          "test_quantize_key_matches_workload_recipe"]),
    ("indexer_scores_row", _no_relu, ["test_indexer_one_hot_keys_read_out_query_columns",
                                      "test_indexer_single_head_relu_of_dot"]),
    ("indexer_scores_row", _reversed_head_weights, ["test_indexer_one_hot_keys_read_out_query_columns"]),
    ("indexer_scores_row", _relu_after_sum, ["test_indexer_one_hot_keys_read_out_query_columns"]),
    ("indexer_scores", _causal_off_by_one, ["test_indexer_causal_multi_query",
                                            "test_mla_all_positions_equals_dense_causal_attention"]),
    ("topk_row", _reversed_ties, ["test_topk_all_equal_scores_take_lowest_positions",
                                  "test_topk_brute_force_and_invariants"]),
    ("sparse_mla_row", _unscaled_mla, ["test_mla_all_positions_equals_dense_causal_attention",
                                       "test_mla_absorption_identity"]),
    ("sparse_mla_row", _value_with_rope, ["test_mla_value_excludes_rope_part",
                                          "test_mla_all_positions_equals_dense_causal_attention"]),
    ("physical_slots", _no_block_table, ["test_indexer_block_table_invariance"]),
    ("physical_slots", _wrong_sequence_table, ["test_indexer_block_table_invariance"]),
    ("indexer_keys", _fp8_scale_ignored, ["test_indexer_fp8_equals_bf16_on_representable_keys"]),
    ("e4m3fn_to_f64", _e4m3_fnuz, ["test_indexer_fp8_equals_bf16_on_representable_keys"]),
]


def _call(name):
    fn = getattr(pins, name)
    if name == "test_topk_brute_force_and_invariants":
        return fn(64, 16)
    if name == "test_page_budget_worked_example":
        return fn(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
    return fn()


@pytest.mark.parametrize("target,mutant,caught_by", MUTATIONS,
                         ids=[f"{t}:{m.__name__}" for t, m, _ in MUTATIONS])
def test_mutation_is_caught(monkeypatch, target, mutant, caught_by):
    for name in caught_by:
        _call(name)  # passes on the real oracle
    monkeypatch.setattr(O, target, mutant)
    for name in caught_by:
        with pytest.raises((AssertionError, ValueError, IndexError)):
            _call(name)
