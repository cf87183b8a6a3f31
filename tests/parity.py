"""Shared helpers of the GPU parity tests: run the HIP path through the binding,
run the oracle on the same seeded inputs, and compare at the documented bars.

Tolerances (fixed by the method's statement of accuracy):
* indexer scores and attention outputs: max |GPU - oracle| <= 1e-2 * RMS(oracle);
* top-k given identical scores: bit-exact;
* top-k end to end: the two selections may differ only at positions whose
  oracle score lies within 1e-3 * |k-th oracle score| of the k-th score.
"""

from __future__ import annotations

import numpy as np
import torch

import sparse_attention_decode_lightning_amd as dsa
from oracle import dsa_oracle as O
from workloads import host_view

SCORE_TOL = 1e-2
OUT_TOL = 1e-2
BAND = 1e-3
LSE_TOL = 1e-4


def batch_of(inp) -> dsa.Batch:
    return dsa.Batch(inp.block_table, inp.seq_lens, inp.cu_q, inp.total_q, inp.max_seq_len,
                     inp.max_q)


def keys_of(inp) -> dsa.PagedCache:
    return dsa.PagedCache(inp.k_cache, inp.k_scale)


def run_gpu(inp, canary: bool = True):
    """Whole pass on the GPU; outputs are pre-filled with NaN / sentinels so untouched
    entries are visible, and each output has a guard row that must stay intact."""
    wl = inp.wl
    dev = inp.q_idx.device
    T = inp.total_q
    ld = max(1, inp.max_seq_len)
    g = 1 if canary else 0
    scores = torch.full((T + g, ld), float("nan"), dtype=torch.float32, device=dev)
    indices = torch.full((T + g, wl.topk), 0x7EADBEEF, dtype=torch.int32, device=dev)
    b = batch_of(inp)
    dsa.indexer_scores(b, inp.q_idx, inp.w, keys_of(inp), scores=scores[:T])
    dsa.topk(b, scores[:T], wl.topk, indices=indices[:T])
    outs = []
    for l in range(wl.n_layers):
        out = torch.full((T + g, wl.mla_heads, wl.d_latent), float("nan"), dtype=torch.float32,
                         device=dev)
        lse = torch.full((T + g, wl.mla_heads), float("nan"), dtype=torch.float32, device=dev)
        dsa.sparse_mla_fwd(b, inp.q_mla[l], dsa.PagedCache(inp.kv_cache[l]), indices[:T],
                           wl.d_latent, wl.scale, out=out[:T], lse=lse[:T])
        outs.append((out, lse))
    torch.cuda.synchronize()
    if canary:
        assert torch.isnan(scores[T]).all(), "write past the scores buffer"
        assert (indices[T] == 0x7EADBEEF).all(), "write past the indices buffer"
        for out, lse in outs:
            assert torch.isnan(out[T]).all() and torch.isnan(lse[T]).all(), "write past out/lse"
    return scores[:T], indices[:T], [(o[:T], s[:T]) for o, s in outs]


def positions(inp):
    return O.row_positions(inp.seq_lens_host, inp.q_lens_host)


def check_scores(inp, gpu_scores, rows, host=None):
    """Valid region equal to the oracle within 1e-2 RMS; entries past t untouched (NaN)."""
    host = host or host_view(inp, lazy=True)
    ref = O.indexer_scores(host, rows)
    _, pos = positions(inp)
    g = gpu_scores[list(rows)].double().cpu().numpy()
    errs, sq, n = [], 0.0, 0
    for i, r in enumerate(rows):
        t = int(pos[r])
        got = g[i, : t + 1]
        assert np.isfinite(got).all(), f"row {r}: non-finite score in the valid region"
        assert np.isnan(g[i, t + 1:]).all(), f"row {r}: wrote past its causal bound"
        errs.append(np.max(np.abs(got - ref[r])))
        sq += float(np.sum(ref[r] ** 2))
        n += ref[r].size
    rms = np.sqrt(sq / max(n, 1))
    assert max(errs) <= SCORE_TOL * rms, (max(errs), rms)
    return ref


def check_topk_identical(gpu_scores, gpu_idx, rows, inp, k):
    """Oracle top-k of the GPU's own fp32 scores equals the GPU's indices exactly."""
    _, pos = positions(inp)
    s = gpu_scores[list(rows)].double().cpu().numpy()
    gi = gpu_idx[list(rows)].cpu().numpy()
    for i, r in enumerate(rows):
        t = int(pos[r])
        ref = O.topk_row(s[i, : t + 1], k)
        assert np.array_equal(gi[i], ref), f"row {r}: top-k differs on identical scores"


def check_topk_band(ref_scores, gpu_idx, rows, k):
    """End to end: selections differ only inside the 1e-3 band around the k-th oracle score."""
    gi = gpu_idx[list(rows)].cpu().numpy()
    for i, r in enumerate(rows):
        s = ref_scores[r]
        ref = O.topk_row(s, k)
        a = set(int(x) for x in ref if x >= 0)
        b = set(int(x) for x in gi[i] if x >= 0)
        assert len(a) == len(b)
        if a == b:
            continue
        kth = np.sort(s)[::-1][min(k, len(s)) - 1]
        for p in a ^ b:
            assert abs(s[p] - kth) <= BAND * abs(kth), (r, p, s[p], kth)


def check_invariants(inp, gpu_idx, k):
    """Every row: ascending unique positions in [0, t], count min(k, t+1), then -1."""
    _, pos = positions(inp)
    idx = gpu_idx.cpu().numpy()
    for r in range(idx.shape[0]):
        n = min(k, int(pos[r]) + 1)
        row = idx[r]
        assert (row[n:] == -1).all(), f"row {r}: bad padding"
        sel = row[:n]
        assert (sel >= 0).all() and (sel <= pos[r]).all(), f"row {r}: non-causal index"
        assert (np.diff(sel) > 0).all(), f"row {r}: not strictly ascending"


def check_mla(inp, layer, gpu_idx, out, lse, rows, host=None):
    """Oracle MLA on the GPU's own indices; max error <= 1e-2 RMS over the checked rows."""
    host = host or host_view(inp, lazy=True)
    idx = gpu_idx[list(rows)].cpu().numpy()
    ref = O.sparse_mla(host, layer, {r: idx[i] for i, r in enumerate(rows)})
    o = out[list(rows)].double().cpu().numpy()
    s = lse[list(rows)].double().cpu().numpy()
    ro = np.stack([ref[r][0] for r in rows])
    rl = np.stack([ref[r][1] for r in rows])
    assert np.isfinite(o).all()
    rms = np.sqrt(np.mean(ro ** 2))
    err = np.max(np.abs(o - ro))
    assert err <= OUT_TOL * rms, (err, rms)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(s))
    assert np.all(np.abs(s[fin] - rl[fin]) <= LSE_TOL * np.maximum(1.0, np.abs(rl[fin])))
    return err, rms
