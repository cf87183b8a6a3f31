"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test pins one step of the oracle to a closed form, an invariant, a
library routine, brute force on a tiny input, or a value the pages print, so
that a plausible mistake (a dropped ReLU, transposed heads and dims, a wrong
page lookup, an off-by-one causal bound, a reversed tie rule, a missing
scale, the RoPE part leaking into the value) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from workloads import WORKLOADS, host_view, make_inputs, small_variant

RNG = np.random.default_rng(1234)


# --------------------------------------------------------------------------
# helpers: hand-built host inputs (f32 storage unless stated)
# --------------------------------------------------------------------------


def make_host(keys_per_seq, q_idx, w, page_size=4, shuffle=True, seed=0, kv_rows=None,
              q_mla=None, q_lens=None, k_dtype="f32", k_scale_per_seq=None, topk=4,
              d_latent=None, scale=0.25):
    """Pack per-sequence logical key arrays [L_b, D] into a shuffled paged pool."""
    rng = np.random.default_rng(seed)
    B = len(keys_per_seq)
    lens = [k.shape[0] for k in keys_per_seq]
    q_lens = q_lens or [1] * B
    pages = [(L + page_size - 1) // page_size for L in lens]
    pool = sum(pages) + 2
    perm = rng.permutation(pool) if shuffle else np.arange(pool)
    bt = np.zeros((B, max(pages)), dtype=np.int32)
    D = keys_per_seq[0].shape[1]
    kdt = np.uint8 if k_dtype == "fp8" else np.float32
    kc = np.zeros((pool, page_size, D), dtype=kdt)
    ks = np.ones((pool, page_size), dtype=np.float32)
    kv = None
    if kv_rows is not None:
        kv = np.zeros((pool, page_size, kv_rows[0].shape[1]), dtype=np.float32)
    off = 0
    for b in range(B):
        bt[b, : pages[b]] = perm[off: off + pages[b]]
        off += pages[b]
        for s in range(lens[b]):
            p, sl = bt[b, s // page_size], s % page_size
            kc[p, sl] = keys_per_seq[b][s]
            if k_scale_per_seq is not None:
                ks[p, sl] = k_scale_per_seq[b][s]
            if kv is not None:
                kv[p, sl] = kv_rows[b][s]
    h = {
        "seq_lens": lens, "q_lens": q_lens, "block_table": bt, "page_size": page_size,
        "q_idx": np.asarray(q_idx, dtype=np.float32), "idx_q_dtype": "f32",
        "w": np.asarray(w, dtype=np.float32), "k_cache": kc,
        "k_scale": ks if k_dtype == "fp8" else None, "idx_k_dtype": k_dtype,
        "q_mla": [] if q_mla is None else [np.asarray(q_mla, dtype=np.float32)],
        "kv_cache": [] if kv is None else [kv], "mla_dtype": "f32",
        "d_latent": d_latent, "scale": scale, "topk": topk,
    }
    return h


# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------


def test_e4m3fn_table_matches_torch_for_all_codes():
    """The table built from the format definition equals torch's float8_e4m3fn decode."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = O.e4m3fn_table()
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(tab[ok], ref[ok])
    assert np.array_equal(np.signbit(tab[ok]), np.signbit(ref[ok]))


def test_e4m3fn_known_codes():
    tab = O.e4m3fn_table()
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x08] == 2.0 ** -6  # smallest normal
    assert tab[0x01] == 2.0 ** -9  # smallest subnormal
    assert tab[0x07] == 7 * 2.0 ** -9
    assert tab[0x38] == 1.0
    assert tab[0x00] == 0.0 and np.signbit(tab[0x80])
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert np.sum(np.isnan(tab)) == 2  # no other NaN, no infinity
    assert np.all(np.isfinite(tab[~np.isnan(tab)]))


def test_bf16_decode_matches_torch():
    x = torch.tensor(RNG.standard_normal(4096) * 10.0 ** RNG.integers(-30, 30, 4096),
                     dtype=torch.float32).to(torch.bfloat16)
    x = torch.cat([x, torch.tensor([0.0, -0.0, float("inf"), -float("inf")], dtype=torch.bfloat16)])
    bits = x.view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_to_f64(bits)
    ref = x.to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


# --------------------------------------------------------------------------
# positions
# --------------------------------------------------------------------------


def test_row_positions_absolute():
    """Row i of a sequence with q new tokens and total length L sits at L - q + i."""
    seq, pos = O.row_positions([10, 7, 5], [3, 1, 0])
    assert seq.tolist() == [0, 0, 0, 1]
    assert pos.tolist() == [7, 8, 9, 6]


# --------------------------------------------------------------------------
# indexer
# --------------------------------------------------------------------------


def test_indexer_zero_query_gives_zero():
    keys = [RNG.standard_normal((13, 8))]
    h = make_host(keys, np.zeros((1, 3, 8)), RNG.standard_normal((1, 3)))
    s = O.indexer_scores(h)[0]
    assert s.shape == (13,) and np.all(s == 0.0)


def test_indexer_one_hot_keys_read_out_query_columns():
    """Key s = unit vector e_d gives sum_j w_j * max(0, q[j, d]): pins heads vs dims and the ReLU."""
    H, D = 5, 7
    q = RNG.standard_normal((1, H, D))
    w = RNG.standard_normal((1, H))
    dims = [3, 0, 6, 2, 2, 5, 1, 4, 6]
    keys = np.zeros((len(dims), D))
    for s, d in enumerate(dims):
        keys[s, d] = 1.0
    h = make_host([keys], q, w, page_size=2)
    s = O.indexer_scores(h)[0]
    qf = q.astype(np.float32).astype(np.float64)[0]
    wf = w.astype(np.float32).astype(np.float64)[0]
    for si, d in enumerate(dims):
        expect = sum(wf[j] * max(0.0, qf[j, d]) for j in range(H))
        assert s[si] == pytest.approx(expect, rel=1e-15, abs=1e-15)


def test_indexer_single_head_relu_of_dot():
    """H_I = 1, w = 1: k = q gives |q|^2, k = -q gives 0 (ReLU), k = 2q gives 2|q|^2."""
    D = 16
    q = np.float32(RNG.standard_normal((1, 1, D))).astype(np.float64)
    keys = np.stack([q[0, 0], -q[0, 0], 2 * q[0, 0], np.zeros(D)])
    h = make_host([keys], q, np.ones((1, 1)))
    s = O.indexer_scores(h)[0]
    n2 = float(np.dot(q[0, 0], q[0, 0]))
    assert s[0] == pytest.approx(n2, rel=1e-14)
    assert s[1] == 0.0
    assert s[2] == pytest.approx(2 * n2, rel=1e-14)
    assert s[3] == 0.0


def test_indexer_brute_force_tiny():
    """Pure-Python loops over (key, head, dim) agree with the vectorized oracle on the tiny workload."""
    inp = make_inputs(WORKLOADS["tiny"])
    h = host_view(inp)
    s = O.indexer_scores(h)[0]
    q = h["q_idx"].astype(np.float64)[0]
    w = h["w"].astype(np.float64)[0]
    bt, P = h["block_table"], h["page_size"]
    L = h["seq_lens"][0]
    assert s.shape == (L,)
    for pos in range(L):
        key = h["k_cache"][bt[0, pos // P], pos % P].astype(np.float64)
        tot = 0.0
        for j in range(q.shape[0]):
            d = math.fsum(float(q[j, i]) * float(key[i]) for i in range(q.shape[1]))
            tot += float(w[j]) * max(0.0, d)
        assert s[pos] == pytest.approx(tot, rel=1e-12, abs=1e-12)


def test_indexer_block_table_invariance():
    """An identity and a shuffled page table over the same logical keys give identical scores."""
    keys = [RNG.standard_normal((37, 8)), RNG.standard_normal((21, 8))]
    q = RNG.standard_normal((2, 3, 8))
    w = RNG.standard_normal((2, 3))
    a = O.indexer_scores(make_host(keys, q, w, page_size=4, shuffle=False))
    b = O.indexer_scores(make_host(keys, q, w, page_size=4, shuffle=True, seed=7))
    for r in (0, 1):
        assert np.array_equal(a[r], b[r])
    # and the second sequence reads its own keys, not the first one's
    c = O.indexer_scores(make_host([keys[1], keys[0]], q[::-1], w[::-1], page_size=4))
    assert np.array_equal(c[0], a[1]) and np.array_equal(c[1], a[0])


def test_indexer_causal_multi_query():
    """Query i of q new tokens sees exactly positions 0..L-q+i; later keys do not change its scores."""
    L, qn = 19, 4
    keys = RNG.standard_normal((L, 6))
    q = RNG.standard_normal((qn, 2, 6))
    w = RNG.standard_normal((qn, 2))
    s1 = O.indexer_scores(make_host([keys], q, w, q_lens=[qn]))
    keys2 = keys.copy()
    keys2[L - qn + 1:] = 1e6  # changes only keys later than the first query
    s2 = O.indexer_scores(make_host([keys2], q, w, q_lens=[qn]))
    for i in range(qn):
        assert s1[i].shape == (L - qn + i + 1,)
    assert np.array_equal(s1[0], s2[0])
    assert not np.array_equal(s1[qn - 1], s2[qn - 1])


def test_indexer_fp8_equals_bf16_on_representable_keys():
    """Keys exactly representable in e4m3fn: fp8 storage with sigma = 1 equals float storage; sigma = 2^-3 scales exactly."""
    tab = O.e4m3fn_table()
    finite = np.where(np.isfinite(tab) & (np.abs(tab) < 64))[0]
    codes = RNG.choice(finite, size=(30, 16)).astype(np.uint8)
    vals = tab[codes]
    q = RNG.standard_normal((1, 4, 16))
    w = RNG.standard_normal((1, 4))
    a = O.indexer_scores(make_host([vals], q, w))[0]
    b = O.indexer_scores(make_host([codes], q, w, k_dtype="fp8",
                                   k_scale_per_seq=[np.ones(30, np.float32)]))[0]
    assert np.array_equal(a, b)
    c = O.indexer_scores(make_host([codes], q, w, k_dtype="fp8",
                                   k_scale_per_seq=[np.full(30, 0.125, np.float32)]))[0]
    assert np.allclose(c, a * 0.125, rtol=1e-14, atol=0)


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------


def brute_topk(scores, k):
    order = sorted(range(len(scores)), key=lambda s: (-float(scores[s]), s))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


def check_topk_invariants(scores, idx, k):
    sel = [int(x) for x in idx if x >= 0]
    n = len(scores)
    assert len(sel) == min(k, n)
    assert all(x == -1 for x in idx[len(sel):])
    assert sel == sorted(set(sel))  # unique, ascending
    assert all(0 <= x < n for x in sel)  # causal
    chosen = set(sel)
    rest = [s for s in range(n) if s not in chosen]
    if rest and sel:
        lo = min(scores[s] for s in sel)
        hi = max(scores[s] for s in rest)
        assert lo >= hi  # maximal
        if lo == hi:  # ties broken toward lower positions
            assert max(s for s in sel if scores[s] == lo) < min(s for s in rest if scores[s] == hi)


@pytest.mark.parametrize("n,k", [(1, 4), (5, 4), (64, 16), (257, 64), (300, 300), (40, 64)])
def test_topk_brute_force_and_invariants(n, k):
    s = np.round(RNG.standard_normal(n) * 4) / 4  # many ties
    got = O.topk_row(s, k)
    assert got.tolist() == brute_topk(s, k)
    check_topk_invariants(s, got, k)


def test_topk_all_equal_scores_take_lowest_positions():
    got = O.topk_row(np.zeros(100), 10)
    assert got.tolist() == list(range(10))


def test_topk_signed_zeros_are_equal():
    s = np.array([0.0, -0.0, 0.0, -0.0, -1.0, -0.0, 0.0])
    assert O.topk_row(s, 3).tolist() == [0, 1, 2]
    s2 = np.array([-0.0, 0.0, -0.0, 0.0])
    assert O.topk_row(s2, 2).tolist() == [0, 1]


def test_topk_fewer_candidates_than_k():
    s = RNG.standard_normal(7)
    assert O.topk_row(s, 10).tolist() == list(range(7)) + [-1] * 3


def test_topk_tiny_workload():
    h = host_view(make_inputs(WORKLOADS["tiny"]))
    s = O.indexer_scores(h)
    idx = O.topk(s, h["topk"])
    assert idx[0].tolist() == brute_topk(s[0], h["topk"])
    check_topk_invariants(s[0], idx[0], h["topk"])


# --------------------------------------------------------------------------
# sparse MLA
# --------------------------------------------------------------------------


def sdpa64(q, k, v, scale, mask=None):
    """torch scaled_dot_product_attention in float64 on the CPU (library routine)."""
    tq = torch.tensor(q, dtype=torch.float64)
    tk = torch.tensor(k, dtype=torch.float64)
    tv = torch.tensor(v, dtype=torch.float64)
    m = None if mask is None else torch.tensor(mask)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale).numpy()


def test_mla_all_positions_equals_dense_causal_attention():
    """k >= L: selecting every causal position reduces to dense causal attention (torch SDPA, float64)."""
    H, DL, DR, L, qn = 4, 24, 8, 29, 3
    rows = RNG.standard_normal((L, DL + DR))
    qm = RNG.standard_normal((qn, H, DL + DR))
    keys = RNG.standard_normal((L, 4))
    h = make_host([keys], RNG.standard_normal((qn, 2, 4)), RNG.standard_normal((qn, 2)),
                  kv_rows=[rows], q_mla=qm, q_lens=[qn], topk=64, d_latent=DL, scale=0.3)
    s = O.indexer_scores(h)
    idx = O.topk(s, 64)
    out = O.sparse_mla(h, 0, idx)
    rf = rows.astype(np.float32).astype(np.float64)
    qf = qm.astype(np.float32).astype(np.float64)
    sc = float(np.float32(0.3))
    mask = np.zeros((qn, L), dtype=bool)
    for i in range(qn):
        mask[i, : L - qn + i + 1] = True
    for hh in range(H):
        ref = sdpa64(qf[:, hh], rf, rf[:, :DL], sc, mask)
        for i in range(qn):
            assert np.allclose(out[i][0][hh], ref[i], rtol=1e-12, atol=1e-13)


def test_mla_absorption_identity():
    """Absorbed MLA (576-d q over latent|rope rows, value = latent) equals explicit per-head
    attention with k = [W_UK c ; k_rope], v = W_UV c and scale 1/sqrt(192 + 64), after W_UV."""
    H, DN, DRo, DV, DC, n = 3, 192, 64, 256, 512, 40
    W_UK = RNG.standard_normal((H, DN, DC)) / math.sqrt(DC)
    W_UV = RNG.standard_normal((H, DV, DC)) / math.sqrt(DC)
    c = RNG.standard_normal((n, DC))
    kr = RNG.standard_normal((n, DRo))
    q_nope = RNG.standard_normal((H, DN))
    q_rope = RNG.standard_normal((H, DRo))
    scale = 1.0 / math.sqrt(DN + DRo)
    rows = np.concatenate([c, kr], axis=1)
    q_abs = np.stack([np.concatenate([W_UK[hh].T @ q_nope[hh], q_rope[hh]]) for hh in range(H)])
    o_abs, _ = O.sparse_mla_row(q_abs, rows, scale, DC)
    for hh in range(H):
        k_h = np.concatenate([c @ W_UK[hh].T, kr], axis=1)  # [n, 256]
        v_h = c @ W_UV[hh].T  # [n, 256]
        q_h = np.concatenate([q_nope[hh], q_rope[hh]])[None]
        ref = sdpa64(q_h, k_h, v_h, scale)[0]
        assert np.allclose(W_UV[hh] @ o_abs[hh], ref, rtol=1e-10, atol=1e-12)


def test_mla_identical_rows_and_zero_query():
    H, DL, n = 3, 10, 7
    row = RNG.standard_normal(DL + 4)
    o, lse = O.sparse_mla_row(RNG.standard_normal((H, DL + 4)), np.tile(row, (n, 1)), 0.5, DL)
    assert np.allclose(o, np.tile(row[:DL], (H, 1)), rtol=1e-14, atol=1e-14)
    rows = RNG.standard_normal((n, DL + 4))
    o0, lse0 = O.sparse_mla_row(np.zeros((H, DL + 4)), rows, 0.5, DL)
    assert np.allclose(o0, np.tile(rows[:, :DL].mean(0), (H, 1)), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse0, math.log(n), rtol=1e-15)


def test_mla_padding_and_permutation():
    """-1 entries are dropped; the order of the selected positions does not matter."""
    H, DL, DR, L = 2, 12, 4, 16
    rows = RNG.standard_normal((L, DL + DR))
    qm = RNG.standard_normal((1, H, DL + DR))
    h = make_host([RNG.standard_normal((L, 3))], RNG.standard_normal((1, 1, 3)),
                  np.ones((1, 1)), kv_rows=[rows], q_mla=qm, d_latent=DL, topk=8)
    a = O.sparse_mla(h, 0, {0: np.array([1, 4, 9, 15, -1, -1, -1, -1])})[0]
    b = O.sparse_mla(h, 0, {0: np.array([15, -1, 9, 1, -1, 4, -1, -1])})[0]
    assert np.allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    assert np.allclose(a[1], b[1], rtol=1e-14)
    e = O.sparse_mla(h, 0, {0: np.full(8, -1)})[0]
    assert np.all(e[0] == 0) and np.all(np.isneginf(e[1]))


def test_mla_value_excludes_rope_part():
    """Changing only the RoPE key part of a row changes the weights, never the value vector."""
    H, DL, DR, n = 2, 6, 3, 5
    rows = RNG.standard_normal((n, DL + DR))
    q = np.zeros((H, DL + DR))
    rows2 = rows.copy()
    rows2[:, DL:] = 1e3
    a, _ = O.sparse_mla_row(q, rows, 1.0, DL)
    b, _ = O.sparse_mla_row(q, rows2, 1.0, DL)  # q = 0 -> uniform weights either way
    assert np.allclose(a, b, rtol=1e-14)


def test_pipeline_topk_at_least_length_is_dense_attention():
    """End to end on a small batch with k >= L: the output is dense causal MLA whatever the indexer says."""
    wl = small_variant("tiny", batch=2, lens=(37, 20), q_per_seq=(2, 1), topk=64)
    inp = make_inputs(wl)
    h = host_view(inp)
    _, idx, outs = O.run(h)
    out = outs[0]
    seq, pos = O.row_positions(h["seq_lens"], h["q_lens"])
    P, bt = h["page_size"], h["block_table"]
    for r in range(len(seq)):
        b, t = int(seq[r]), int(pos[r])
        rows = np.stack([h["kv_cache"][0][bt[b, s // P], s % P] for s in range(t + 1)]).astype(np.float64)
        q = h["q_mla"][0][r].astype(np.float64)
        ref = sdpa64(q, rows, rows[:, : h["d_latent"]], float(np.float32(h["scale"])))
        assert np.allclose(out[r][0], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# IndexShare
# --------------------------------------------------------------------------


def test_indexshare_pattern_matches_printed_string(golden_dir):
    lines = [ln.strip() for ln in open(os.path.join(golden_dir, "glm52_index_topk_pattern.txt"))
             if ln.strip() and not ln.startswith("#")]
    printed = lines[0]
    assert len(printed) == 78 and printed.count("F") == 21 and printed.count("S") == 57
    assert O.glm52_indexer_pattern(78) == printed
    owner = O.indexer_owner_layers(printed)
    assert owner[:8] == [0, 1, 2, 2, 2, 2, 6, 6]
    assert owner[77] == 74
    assert all(printed[o] == "F" for o in owner)


def test_indexshare_rejects_shared_layer_without_owner():
    with pytest.raises(ValueError):
        O.indexer_owner_layers("SFF")


# --------------------------------------------------------------------------
# paged append: e4m3 quantisation and the slot scatter
# --------------------------------------------------------------------------


def _e4m3_edge_values() -> np.ndarray:
    """Every finite e4m3 value, every midpoint of two neighbours, and the floats beside them."""
    tab = O.e4m3fn_table()
    mags = np.sort(tab[:0x7F]).astype(np.float32)
    mids = ((mags[:-1].astype(np.float64) + mags[1:]) / 2).astype(np.float32)  # exact in fp32
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(448))])
    vals = np.concatenate([mags, mids, near, [2.0 ** -12, 2.0 ** -10, 1e-30, 447.99]])
    return np.concatenate([vals, -vals, [0.0, -0.0]]).astype(np.float32)


def test_e4m3_encode_matches_torch_cast():
    """Library routine: torch's float8_e4m3fn conversion rounds to nearest, ties to even."""
    rng = np.random.default_rng(7)
    rand = rng.standard_normal(3000) * rng.choice([1e-3, 0.05, 1.0, 40.0, 300.0], 3000)
    x = np.concatenate([_e4m3_edge_values(), np.clip(rand, -448, 448)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3fn_encode(x), ref)


def test_e4m3_encode_round_trip_and_ties_to_even():
    """Closed form: a code's own value encodes to it; a midpoint goes to the even code."""
    tab = O.e4m3fn_table()
    for c in range(256):
        if not np.isnan(tab[c]):
            v = np.float32(-0.0) if c == 0x80 else np.float32(tab[c])
            assert int(O.e4m3fn_encode(v)) == c, hex(c)
    for c in range(0x7E):  # neighbours c, c + 1 among the positive codes
        mid = np.float32((tab[c] + tab[c + 1]) / 2)
        want = c if c % 2 == 0 else c + 1
        assert int(O.e4m3fn_encode(mid)) == want
        assert int(O.e4m3fn_encode(-mid)) == want | 0x80


def test_quantize_key_scale_and_error_bound():
    """sigma = max|k| / 448 in fp32; the largest element lands on +-448; every element is
    within half an e4m3 step (2^-4 relative, or sigma 2^-10 in the subnormal range)."""
    rng = np.random.default_rng(8)
    for _ in range(20):
        k = (rng.standard_normal(128) * rng.choice([1e-3, 1.0, 50.0])).astype(np.float32)
        codes, sigma = O.quantize_key_e4m3(k)
        assert sigma == np.float32(np.abs(k).max()) / np.float32(448.0)
        assert int(codes[np.argmax(np.abs(k))]) & 0x7F == 0x7E
        deq = np.float64(sigma) * O.e4m3fn_table()[codes]
        bound = np.maximum(np.abs(k) * 2.0 ** -4, float(sigma) * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(deq - k) <= bound)
    z, s0 = O.quantize_key_e4m3(np.zeros(128, np.float32))
    assert s0 == np.float32(1.0) and not z.any()


def test_quantize_key_matches_workload_recipe():
    """The workload generator's torch recipe (amax / 448, clamp, float8 cast) and the oracle
    give the same bytes and scales."""
    g = torch.Generator().manual_seed(9)
    k = torch.randn((64, 128), generator=g) * torch.rand((64, 1), generator=g) * 10
    sig = k.abs().amax(dim=-1) / 448.0
    ref = (k / sig[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i in range(64):
        codes, sigma = O.quantize_key_e4m3(k[i].numpy())
        assert sigma == np.float32(sig[i].item())
        assert np.array_equal(codes, ref[i])


def test_kv_append_writes_only_mapped_slots():
    """Invariant: mapped slots take the new rows, skipped tokens (negative or out-of-pool
    slots) and every other slot keep their bytes; fp8 keys carry their scale."""
    rng = np.random.default_rng(10)
    pages, P, R, D = 5, 4, 12, 8
    kv = rng.integers(0, 1 << 15, (pages, P, R), dtype=np.uint16)
    keys = rng.integers(0, 0x7F, (pages, P, D), dtype=np.uint8)
    scale = rng.random((pages, P)).astype(np.float32)
    slots = np.array([7, -1, pages * P, 0, 19, -3], dtype=np.int32)
    lat = rng.integers(0, 1 << 15, (6, R), dtype=np.uint16)
    new_k = rng.standard_normal((6, D)).astype(np.float32)
    kv2, keys2, scale2 = O.kv_append(slots, lat, kv, new_k, keys, scale, key_cache_dtype="fp8")
    written = {7: 0, 0: 3, 19: 4}
    for s in range(pages * P):
        p, o = divmod(s, P)
        if s in written:
            i = written[s]
            assert np.array_equal(kv2[p, o], lat[i])
            codes, sigma = O.quantize_key_e4m3(new_k[i])
            assert np.array_equal(keys2[p, o], codes) and scale2[p, o] == sigma
        else:
            assert np.array_equal(kv2[p, o], kv[p, o])
            assert np.array_equal(keys2[p, o], keys[p, o]) and scale2[p, o] == scale[p, o]
    kv3, keys3, _ = O.kv_append(slots, lat, kv, new_k.astype(np.float32), keys, None,
                                key_cache_dtype="f32")
    assert keys3.dtype == keys.dtype and np.array_equal(kv3, kv2)


# --------------------------------------------------------------------------
# page-budget selection
# --------------------------------------------------------------------------


def _golden_page_example(golden):
    d = {}
    for ln in open(os.path.join(golden, "page_budget_example.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        key, *vals = ln.split()
        d[key] = [float(v) for v in vals]
    return d


def test_page_budget_worked_example(golden_dir):
    """The pages' printed example: token top-4 names four positions, expanding their pages
    reads sixteen, a two-page budget reads eight (tests/golden/page_budget_example.txt)."""
    d = _golden_page_example(golden_dir)
    P, k, kp = int(d["page_size"][0]), int(d["token_topk"][0]), int(d["page_budget"][0])
    s = np.array(d["scores"])
    tok = O.topk_row(s, k)
    assert list(tok) == [int(v) for v in d["token_positions"]]
    assert len({int(p) // P for p in tok}) * P == int(d["expanded_pages_reads"][0])
    pages, idx = O.page_budget_select({0: s}, P, kp)
    assert list(pages[0]) == [int(v) for v in d["budget_pages"]]
    assert int((idx[0] >= 0).sum()) == int(d["budget_reads"][0])
    assert list(idx[0]) == [p * P + o for p in pages[0] for o in range(P)]


def test_page_budget_brute_force_with_masked_future():
    """Brute force on tiny rows: a page's score is the maximum of its positions <= t only
    (a huge score past t must not promote its page); kp best pages by (score desc, page asc)."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        P = int(rng.choice([1, 2, 4, 8]))
        L = int(rng.integers(1, 40))
        t = int(rng.integers(0, L))
        kp = int(rng.integers(1, 6))
        full = rng.choice([0.0, 1.0, 2.0, 3.0], L) + rng.random(L) * (trial % 2)
        full[t + 1:] = 1e30  # positions past t: invisible
        legal = full[: t + 1]
        pages, idx = O.page_budget_select({0: legal}, P, kp)
        n_pages = t // P + 1
        best = []
        for p in range(n_pages):
            m = max(full[s] for s in range(p * P, min((p + 1) * P, L)) if s <= t)
            best.append((-m, p))
        want = sorted(p for _, p in sorted(best)[:kp])
        got = [int(p) for p in pages[0] if p >= 0]
        assert got == want, (trial, P, t, kp)
        assert list(pages[0][len(want):]) == [-1] * (kp - len(want))
        toks = [int(v) for v in idx[0] if v >= 0]
        assert toks == [p * P + o for p in want for o in range(P) if p * P + o <= t]


def test_page_budget_unit_pages_is_token_topk():
    """Special case: pages of one position make page-budget selection token top-k."""
    rng = np.random.default_rng(12)
    for _ in range(10):
        s = rng.standard_normal(int(rng.integers(5, 60)))
        s[rng.integers(0, len(s), 3)] = s[0]  # some ties
        k = int(rng.integers(1, 10))
        pages, idx = O.page_budget_select({0: s}, 1, k)
        assert np.array_equal(pages[0], O.topk_row(s, k))
        assert np.array_equal(idx[0], O.topk_row(s, k))


def test_page_budget_large_budget_reads_every_legal_position():
    """A budget covering every page reads every position 0..t exactly once."""
    s = np.random.default_rng(13).standard_normal(37)
    pages, idx = O.page_budget_select({0: s}, 8, 5)
    assert list(pages[0]) == [0, 1, 2, 3, 4]
    assert [int(v) for v in idx[0] if v >= 0] == list(range(37))
