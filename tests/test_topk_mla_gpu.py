"""GPU checks of dsa_topk and dsa_sparse_mla_fwd on inputs the end-to-end pass does not make.

* Top-k on synthetic score rows with ties (quantized, all equal, +0.0 / -0.0
  mixes) and continuous scores, at row lengths that reach every dispatch path
  (one register block of 8, 16 or 32 keys per thread; 16K or 32K chunks then
  a merge; the LDS chunks for large k). The oracle's stable sort fixes the unique
  answer (ties toward the lower position), so the comparison is exact.
* Sparse MLA on caller-made index lists: repeated positions (counted twice),
  -1 padding, positions past the row's causal bound and past the sequence
  (treated as -1 by the library's contract), on the 64-head MFMA path and on
  the generic path.
"""

import numpy as np
import pytest
import torch

import sparse_attention_decode_lightning_amd as dsa
from oracle import dsa_oracle as O
from tests import parity as P
from workloads import host_view, make_inputs, small_variant, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _score_rows(kind: str, lens, seed: int) -> list:
    g = np.random.default_rng(seed)
    rows = []
    for L in lens:
        if kind == "quantized":
            s = g.integers(0, 8, size=L).astype(np.float32) * 0.25
        elif kind == "equal":
            s = np.full(L, 1.5, dtype=np.float32)
        elif kind == "signed_zero":
            s = np.where(g.random(L) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
            hot = g.choice(L, size=min(L, 37), replace=False)
            s[hot] = g.random(hot.size).astype(np.float32) + 1.0
        else:  # continuous
            s = g.standard_normal(L).astype(np.float32)
        rows.append(s)
    return rows


TOPK_CASES = [
    # (row lengths, k): one register pass with 8, 16 and 32 keys per thread,
    # 16K chunks then a merge (rows to 128K), 32K chunks then a merge (to
    # 512K at k = 2048), and 32K LDS chunks where the merge would take more
    # than 32K survivors (large k)
    ((300, 8192, 5), 2048),
    ((12000, 16384), 2048),
    ((20000, 32768), 2048),
    ((70000, 33000, 1000), 2048),
    ((300000, 140000), 2048),
    ((100000, 50000), 8192),
    ((5000, 64), 64),
    # rows shorter than one wave with k below the row length, on the 256-thread
    # paths (one and four keys per thread) and the 1024-thread one: lanes past
    # the row take part in the block maximum with key 0
    ((47, 30, 63), 20),
    ((47, 200, 900), 20),
    ((47, 1000, 3000), 20),
    ((47, 5), 1),
]


@pytest.mark.parametrize("kind", ["quantized", "equal", "signed_zero", "continuous"])
@pytest.mark.parametrize("lens,k", TOPK_CASES)
def test_topk_ties_every_path(kind, lens, k, dev):
    print(f"[topk] {kind} {lens} k={k}", flush=True)
    rows = _score_rows(kind, lens, seed=len(lens) * 7 + k)
    B = len(lens)
    ld = max(lens)
    scores = torch.full((B, ld), float("nan"), dtype=torch.float32)
    for r, s in enumerate(rows):
        scores[r, : len(s)] = torch.from_numpy(s)
    seq_lens = torch.tensor(lens, dtype=torch.int32)
    cu_q = torch.arange(B + 1, dtype=torch.int32)
    bt = torch.zeros((B, 1), dtype=torch.int32)
    b = dsa.Batch(bt.to(dev), seq_lens.to(dev), cu_q.to(dev), B, ld, 1)
    idx = dsa.topk(b, scores.to(dev), k).cpu().numpy()
    for r, s in enumerate(rows):
        ref = O.topk_row(s.astype(np.float64), k)
        assert np.array_equal(idx[r], ref), f"row {r} (L={len(s)}): differs from the oracle"


def _caller_indices(k, L, rows, seed):
    """Per row: positions drawn from [-3, L + 40), about 10% of them one repeated
    position and 5% set to -1."""
    g = np.random.default_rng(seed)
    sel = g.integers(-3, L + 40, size=(rows, k)).astype(np.int32)
    rep = g.random((rows, k)) < 0.1
    sel[rep] = np.broadcast_to(sel[:, :1], sel.shape)[rep]
    sel[g.random((rows, k)) < 0.05] = -1
    return sel


MLA_INDEX_CASES = {
    # 64 heads, 512 + 64 bf16: the MFMA kernel (one split and several)
    "bf16_mfma": small_variant("decode_b32_l8k", batch=3, lens=(700, 1300, 90), topk=512),
    "bf16_mfma_multiq": small_variant("decode_b32_l8k", batch=2, lens=(2500, 60), q_per_seq=(4, 2),
                                      topk=1024),
    # other shapes: the generic kernel
    "f32_generic_multiq": small_variant("tiny", batch=2, lens=(256, 100), q_per_seq=3, topk=96),
}


@pytest.mark.parametrize("name", list(MLA_INDEX_CASES))
def test_mla_on_caller_indices(name, dev):
    """Entries outside [0, t] are treated as -1 and a repeated position counts twice:
    the GPU runs on the raw list, the oracle on the list with those entries set to -1."""
    wl = MLA_INDEX_CASES[name]
    print(f"[mla-indices] {name}", flush=True)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    host = host_view(inp_h)
    _, pos = O.row_positions(inp_h.seq_lens_host, inp_h.q_lens_host)
    raw = _caller_indices(wl.topk, max(inp_h.seq_lens_host), len(pos), seed=11)
    assert (raw > pos[:, None]).any() and (raw == -1).any()
    out, lse = dsa.sparse_mla_fwd(P.batch_of(inp), inp.q_mla[0], dsa.PagedCache(inp.kv_cache[0]),
                                  torch.from_numpy(raw).to(dev), wl.d_latent, wl.scale)
    torch.cuda.synchronize()
    masked = np.where((raw >= 0) & (raw <= pos[:, None]), raw, -1).astype(np.int32)
    P.check_mla(inp, 0, torch.from_numpy(masked), out, lse, list(range(len(pos))), host)
