"""CPU oracle for the sparse-attention decode path (indexer -> top-k -> sparse MLA).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the
HIP library is checked against. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never calls it and
shares no code with it.

Everything is computed in float64 with numpy, one step at a time, in the order
the pages describe the method:

* "vLLM Inference Path: GLM-5.2 as an Example" (section "DSA Indexer"): 32
  retrieval query heads of width 128 scan one shared key per past token,
  per-head weights combine the heads, and the 2,048 best positions are kept;
  (section "MLA Projections and KV State"): the cache holds a 512-d latent
  plus a 64-d RoPE key per token; (section "Sparse MLA Attention"): attention
  reads only the selected positions and the causal mask still applies.
* "Making GLM-5.2 Sparse on TPUs" (section "Separate the indexer from the
  attention it controls"): each head's query-key dot product goes through a
  ReLU before the heads are combined with per-head weights; in the absorbed
  form the query carries the key projection and the latents themselves are
  the values (the value projection comes after the attention sum); the scale
  comes from the 192 + 64 query/key width rather than from 576. (Section
  "Pack requests and reuse prefixes"): a query at local offset i after a
  prefix of length P sits at absolute position P + i.
* "GLM-5.2 on vLLM Ascend: Request-to-Backend Inference Path" (section "8. The
  SFA backend, step by step"): the new token's keys are written to the paged
  cache before selection, indices are token positions, and the indexer's keys
  live in their own cache, FP8 e4m3 keys carrying an FP32 scale.

Readings where the pages are silent (each also listed in the design notes):

* the formula has no extra 1/sqrt(d), softmax or scale inside the ReLU; any
  scale lives in w;
* the ReLU applies per head before the w-weighted head sum;
* FP8 means OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF NaN) and the key is
  sigma * e4m3(byte);
* a row at absolute position t sees positions 0..t (its own key included);
* top-k keeps min(k, t + 1) positions ordered by score descending, then by
  position ascending; -0.0 equals +0.0; the result is listed in ascending
  position order and padded with -1;
* the softmax runs over the selected positions only; the value is the first
  d_latent entries of the cached row; an empty selection gives O = 0 and
  lse = -inf.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the upper half of an IEEE binary32."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """All 256 OCP E4M3FN codes -> float64, built from the format's definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    encodes subnormals m/8 * 2^(1-7); the all-ones pattern S.1111.111 is NaN and
    there is no infinity (so S.1111.110 = 448 is the largest finite value).
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = math.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3 = e4m3fn_table()


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Raw stored elements -> float64. ``dtype`` is the storage type tag."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(arr)
    if dtype == "fp8":
        return e4m3fn_to_f64(arr)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# paging and positions
# --------------------------------------------------------------------------


def row_positions(seq_lens: Sequence[int], q_lens: Sequence[int]):
    """For each flattened query row: (sequence b, absolute position t).

    Row cu_q[b] + i of a sequence with KV length L_b (this step's q_b new
    tokens included) is the token at absolute position L_b - q_b + i.
    """
    seq, pos = [], []
    for b, (L, q) in enumerate(zip(seq_lens, q_lens)):
        for i in range(q):
            seq.append(b)
            pos.append(L - q + i)
    return np.array(seq, dtype=np.int64), np.array(pos, dtype=np.int64)


def physical_slots(block_table: np.ndarray, b: int, positions: np.ndarray, page_size: int):
    """Logical token positions of sequence b -> (physical page, slot in page)."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = block_table[b, positions // page_size].astype(np.int64)
    return pages, positions % page_size


def gather_rows(cache: np.ndarray, block_table: np.ndarray, b: int, positions, page_size: int):
    """Raw cache rows of sequence b at the given logical positions (no decoding)."""
    pages, slots = physical_slots(block_table, b, positions, page_size)
    return cache[pages, slots]


# --------------------------------------------------------------------------
# step 1: lightning-indexer scores
# --------------------------------------------------------------------------


def indexer_scores_row(q_idx_row: np.ndarray, w_row: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """I[t, s] = sum_j w[t, j] * ReLU(q_idx[t, j] . k_idx[s]) for every key s given.

    q_idx_row: [H_I, D_I] float64; w_row: [H_I] float64; keys: [n, D_I] float64.
    """
    dots = q_idx_row @ keys.T  # [H_I, n]: one dot product per head and key
    return w_row @ np.maximum(dots, 0.0)  # ReLU per head, then the weighted head sum


def indexer_keys(host: dict, b: int, n: int) -> np.ndarray:
    """Decoded indexer keys of sequence b for positions 0..n-1: sigma_s * e4m3(byte) for fp8."""
    pos = np.arange(n)
    raw = gather_rows(host["k_cache"], host["block_table"], b, pos, host["page_size"])
    keys = decode(raw, host["idx_k_dtype"])
    if host["idx_k_dtype"] == "fp8":
        sc = gather_rows(host["k_scale"], host["block_table"], b, pos, host["page_size"])
        keys = keys * np.asarray(sc, dtype=np.float32).astype(np.float64)[:, None]
    return keys


def indexer_scores(host: dict, rows: Optional[Sequence[int]] = None) -> Dict[int, np.ndarray]:
    """Scores of every causal candidate 0..t for each requested row: {row: float64[t + 1]}."""
    seq, pos = row_positions(host["seq_lens"], host["q_lens"])
    rows = range(len(seq)) if rows is None else rows
    q_all = decode(host["q_idx"], host["idx_q_dtype"])
    w_all = np.asarray(host["w"], dtype=np.float32).astype(np.float64)
    out: Dict[int, np.ndarray] = {}
    by_seq: Dict[int, List[int]] = {}
    for r in rows:
        by_seq.setdefault(int(seq[r]), []).append(int(r))
    for b, rs in by_seq.items():
        n = int(max(pos[r] for r in rs)) + 1
        keys = indexer_keys(host, b, n)
        for r in rs:
            t = int(pos[r])
            out[r] = indexer_scores_row(q_all[r], w_all[r], keys[: t + 1])
    return out


# --------------------------------------------------------------------------
# step 2: per-query top-k
# --------------------------------------------------------------------------


def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k token positions of one query row, as int32[k].

    ``scores`` holds the score of every causal candidate 0..t. The min(k, t+1)
    positions with the largest scores are kept; equal scores are ordered by
    position ascending (a stable sort of the negated scores), -0.0 counting as
    +0.0. The kept positions are listed in ascending order, then -1 padding.
    """
    s = np.asarray(scores, dtype=np.float64)
    assert not np.isnan(s).any(), "scores must be finite"
    n = min(k, s.shape[0])
    order = np.argsort(-s, kind="stable")[:n]
    out = np.full(k, -1, dtype=np.int32)
    out[:n] = np.sort(order)
    return out


def topk(scores: Dict[int, np.ndarray], k: int) -> Dict[int, np.ndarray]:
    return {r: topk_row(s, k) for r, s in scores.items()}


# --------------------------------------------------------------------------
# step 3: absorbed sparse MLA over the selected rows
# --------------------------------------------------------------------------


def sparse_mla_row(q_row: np.ndarray, rows: np.ndarray, scale: float, d_latent: int):
    """Absorbed MLA for one query over its selected cache rows.

    q_row: [H, D_L + D_R] (absorbed latent query | RoPE query), rows: [n, D_L + D_R]
    (latent | RoPE key). Per head h: logits l_s = scale * q_h . row_s, p = softmax(l)
    over the n selected rows, O_h = sum_s p_s * row_s[:D_L]; lse_h = log sum_s exp(l_s).
    """
    H = q_row.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, d_latent)), np.full(H, -np.inf)
    logits = scale * (q_row @ rows.T)  # [H, n]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ rows[:, :d_latent]) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def sparse_mla(host: dict, layer: int, indices: Dict[int, np.ndarray]):
    """{row: (O [H, D_L], lse [H])} for one MLA layer, using each row's selected positions.

    Entries equal to -1 are padding and are skipped; every other entry is one
    selected position (a repeated position would simply count twice).
    """
    seq, _ = row_positions(host["seq_lens"], host["q_lens"])
    q_all = host["q_mla"][layer]
    cache = host["kv_cache"][layer]
    d_latent = host["d_latent"]
    scale = float(np.float32(host["scale"]))
    out = {}
    for r, idx in indices.items():
        b = int(seq[r])
        sel = np.asarray(idx, dtype=np.int64)
        sel = sel[sel >= 0]
        raw = gather_rows(cache, host["block_table"], b, sel, host["page_size"])
        rows = decode(raw, host["mla_dtype"]).reshape(len(sel), cache.shape[-1])
        q = decode(q_all[r], host["mla_dtype"])
        out[r] = sparse_mla_row(q, rows, scale, d_latent)
    return out


# --------------------------------------------------------------------------
# the whole pass and IndexShare
# --------------------------------------------------------------------------


def run(host: dict, rows: Optional[Sequence[int]] = None):
    """Indexer -> top-k -> one sparse-MLA call per layer sharing the same indices."""
    s = indexer_scores(host, rows)
    idx = topk(s, host["topk"])
    outs = [sparse_mla(host, l, idx) for l in range(len(host["q_mla"]))]
    return s, idx, outs


def indexer_owner_layers(pattern: str) -> List[int]:
    """IndexShare: for each layer, the layer whose indexer top-k it consumes.

    ``pattern`` has one character per layer, 'F' for a layer that owns an
    indexer and 'S' for a shared layer, which reuses the top-k of the nearest
    preceding full layer ("vLLM Inference Path: GLM-5.2 as an Example",
    section "DSA Indexer"; "Serving GLM-5.2-504B on 8x RTX PRO 6000 GPUs",
    section "Root cause: a missing index_topk_pattern").
    """
    owner, last = [], None
    for i, c in enumerate(pattern):
        if c == "F":
            last = i
        elif c != "S":
            raise ValueError(f"bad pattern character {c!r}")
        if last is None:
            raise ValueError("a shared layer has no preceding full layer")
        owner.append(last)
    return owner


def glm52_indexer_pattern(n_layers: int = 78) -> str:
    """Full indexers at layers 0, 1, 2, 6, 10, 14 and every fourth layer through 74.

    ("vLLM Inference Path: GLM-5.2 as an Example", section "DSA Indexer".)
    """
    full = {0, 1, 2} | set(range(6, 75, 4))
    return "".join("F" if i in full else "S" for i in range(n_layers))


# --------------------------------------------------------------------------
# appending new tokens to the paged caches
# --------------------------------------------------------------------------


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """Finite float32 values in [-448, 448] -> OCP E4M3FN codes (uint8).

    The code whose value is nearest to x, among the finite codes of x's sign;
    at an exact midpoint between two codes the one with an even code (mantissa
    bit 0 clear) wins. +0 and -0 keep their sign. Found by comparing x with
    every finite code value of the decode table, not by bit manipulation.
    """
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1).astype(np.float64)
    mags = _E4M3[:0x7F]  # codes 0x00..0x7E: every finite non-negative value
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        if not (abs(v) <= 448.0):
            raise ValueError("e4m3fn_encode takes finite values in [-448, 448]")
        neg = math.copysign(1.0, v) < 0
        d = np.abs(mags - abs(v))
        near = np.flatnonzero(d == d.min())
        code = int(near[0]) if len(near) == 1 else int(next(c for c in near if c % 2 == 0))
        out[i] = code | (0x80 if neg else 0)
    return out.reshape(x.shape)


def quantize_key_e4m3(k: np.ndarray):
    """One token's indexer key -> (e4m3fn codes, fp32 scale).

    sigma = max|k| / 448 in fp32 (1 for an all-zero key), codes = nearest
    e4m3fn values of clamp(k / sigma, -448, 448) computed in fp32, so that
    sigma * e4m3(code) is the stored key ("GLM-5.2 on vLLM Ascend ...",
    section "7. GLM-5.2 shared-indexer construction": FP8 e4m3 keys with FP32
    scales). The quantised code is an integer decided by floating point, so
    this step uses the stored format's fp32 arithmetic, not float64.
    """
    k = np.asarray(k, dtype=np.float32)
    amax = np.float32(np.max(np.abs(k))) if k.size else np.float32(0.0)
    sigma = amax / np.float32(448.0) if amax > 0 else np.float32(1.0)
    q = np.clip(k / sigma, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return e4m3fn_encode(q), np.float32(sigma)


def kv_append(slot_mapping, latent=None, kv_cache=None, idx_keys=None, key_cache=None,
              key_scale=None, key_cache_dtype: str = "bf16"):
    """Write new tokens into paged caches; returns updated copies (inputs untouched).

    ("GLM-5.2 on vLLM Ascend ...", section "8. The SFA backend, step by step",
    "Write paged cache": the slot mapping scatters new latent rows and indexer
    keys/scales into their physical pages; "Making GLM-5.2 Sparse on TPUs",
    section "Append new KV without moving the resident cache".)

    Caches are raw storage arrays [num_pages, page_size, row]: uint16 for bf16,
    float32 for f32, uint8 for fp8 (with key_scale [num_pages, page_size]).
    Token i lands in slot s = slot_mapping[i] (page s // page_size, offset
    s % page_size); a negative slot or one past the pool skips the token. A
    latent row, or a key row for an f32/bf16 key cache, is stored as given (its
    raw elements); a key row for an fp8 cache is quantised by
    quantize_key_e4m3 from its float32 value.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kv_out = None if kv_cache is None else np.array(kv_cache, copy=True)
    key_out = None if key_cache is None else np.array(key_cache, copy=True)
    scale_out = None if key_scale is None else np.array(key_scale, copy=True)
    for i, s in enumerate(slots):
        if kv_out is not None:
            n_pages, P = kv_out.shape[:2]
            if 0 <= s < n_pages * P:
                kv_out[s // P, s % P] = np.asarray(latent)[i]
        if key_out is not None:
            n_pages, P = key_out.shape[:2]
            if 0 <= s < n_pages * P:
                row = np.asarray(idx_keys)[i]
                if key_cache_dtype == "fp8":
                    vals = row if row.dtype == np.float32 else bf16_to_f64(row).astype(np.float32)
                    codes, sigma = quantize_key_e4m3(vals)
                    key_out[s // P, s % P] = codes
                    scale_out[s // P, s % P] = sigma
                else:
                    key_out[s // P, s % P] = row
    return kv_out, key_out, scale_out


# --------------------------------------------------------------------------
# page-budget selection (an alternative to token top-k)
# --------------------------------------------------------------------------


def page_scores_row(token_scores: np.ndarray, page_size: int) -> np.ndarray:
    """Score of each logical page of one row: the maximum of its legal token scores.

    ("Making GLM-5.2 Sparse on TPUs", section "Make the sparsity unit match the
    memory unit": a page is ranked by its highest legal token score, and the
    causal and valid-length masks apply before the maximum.) ``token_scores``
    holds exactly the legal positions 0..t of the row, so a page's maximum
    never sees a position past t; the last page may be partial.
    """
    s = np.asarray(token_scores, dtype=np.float64)
    n_pages = (len(s) + page_size - 1) // page_size
    return np.array([s[p * page_size:(p + 1) * page_size].max() for p in range(n_pages)])


def expand_pages(pages: np.ndarray, page_size: int, t: int) -> np.ndarray:
    """Token positions read for the selected pages (same section: attention reads every
    legal token of each kept page): slot i * page_size + o holds pages[i] * page_size + o
    when the page is kept (not -1) and the position is <= t, else -1."""
    out = np.full(len(pages) * page_size, -1, dtype=np.int32)
    for i, p in enumerate(pages):
        if p < 0:
            continue
        for o in range(page_size):
            pos = int(p) * page_size + o
            if pos <= t:
                out[i * page_size + o] = pos
    return out


def page_budget_select(scores: Dict[int, np.ndarray], page_size: int, kp: int):
    """Per row: (the kp best pages, ascending, -1 padded; their token positions).

    Pages are ranked by page_scores_row and kept with the token top-k's rule
    (higher score first, equal scores by lower page), then expanded.
    """
    pages, idx = {}, {}
    for r, s in scores.items():
        pr = topk_row(page_scores_row(s, page_size), kp)
        pages[r] = pr
        idx[r] = expand_pages(pr, page_size, len(s) - 1)
    return pages, idx
