"""GPU parity of the query-blocked sparse MLA (dsa_sparse_mla_fwd_qblocked).

The blocked call computes the same attention as dsa_sparse_mla_fwd, so it is
checked against the oracle's sparse_mla on the same indices (1e-2 RMS, lse to
1e-4), and against the per-query call to rounding:

* index lists from the library's top-k (uniform-random selections) and
  locality-shaped lists (blocks of queries drawing from a few shared pages);
* 64 heads (blocks of 4 queries, four head groups), 16 heads (blocks of 4, one
  group) and 8 heads (blocks of 8); query counts that leave partial blocks;
  page sizes 16, 64 and 128; k not a multiple of the 32-row tile;
* the merge's fallback: caller lists with repeats, -1, positions past t and
  unsorted entries, and decode batches whose blocks span sequences;
* a union longer than one row-table chunk, positions past one 32K-position
  membership window; and the restart path (rows scaled
  so late logits exceed the first tile's reference by more than the headroom).
"""

import numpy as np
import pytest
import torch

import sparse_attention_decode_lightning_amd as dsa
from oracle import dsa_oracle as O
from tests import parity as P
from workloads import host_view, locality_indices, make_inputs, small_variant, to_device

pytestmark = pytest.mark.gpu

PREFILL = small_variant("prefill_q4k_l32k", batch=2, lens=(1200, 700), q_per_seq=(37, 21),
                        page_size=64, topk=256)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _run(inp, idx, layer=0):
    wl = inp.wl
    T = inp.total_q
    b = P.batch_of(inp)
    kv = dsa.PagedCache(inp.kv_cache[layer])
    out = torch.full((T + 1, wl.mla_heads, wl.d_latent), float("nan"), device=idx.device)
    lse = torch.full((T + 1, wl.mla_heads), float("nan"), device=idx.device)
    dsa.sparse_mla_fwd_qblocked(b, inp.q_mla[layer], kv, idx, wl.d_latent, wl.scale, out=out[:T],
                                lse=lse[:T])
    ref_o, ref_l = dsa.sparse_mla_fwd(b, inp.q_mla[layer], kv, idx, wl.d_latent, wl.scale)
    torch.cuda.synchronize()
    assert torch.isnan(out[T]).all() and torch.isnan(lse[T]).all(), "write past out/lse"
    return out[:T], lse[:T], ref_o, ref_l


def _check(inp, inp_h, idx_gpu, idx_oracle=None, layer=0):
    out, lse, ref_o, ref_l = _run(inp, idx_gpu, layer)
    rows = list(range(inp.total_q))
    oi = idx_gpu if idx_oracle is None else idx_oracle
    err, rms = P.check_mla(inp, layer, oi, out, lse, rows, host_view(inp_h))
    # the per-query call on the same indices: the same sums in another order
    d = float((out - ref_o).abs().max())
    assert d <= 1e-2 * rms, (d, rms)
    fin = torch.isfinite(ref_l)
    assert torch.equal(fin, torch.isfinite(lse))
    assert float((lse[fin] - ref_l[fin]).abs().max()) <= 1e-4 * max(1.0, float(ref_l[fin].abs().max()))
    return err, rms


CASES = {
    # (workload, selection): top-k of the pipeline's scores or locality-shaped
    "h64_topk": (PREFILL, "topk"),
    "h64_locality": (PREFILL, "locality"),
    "h64_P128_k300": (small_variant(PREFILL, page_size=128, topk=300), "topk"),
    "h16_topk_P16": (small_variant(PREFILL, mla_heads=16, page_size=16, topk=200), "topk"),
    "h8_topk": (small_variant(PREFILL, mla_heads=8, topk=256), "topk"),
    "h8_locality_k17": (small_variant(PREFILL, mla_heads=8, topk=17), "locality"),
    "h32_locality": (small_variant(PREFILL, mla_heads=32, topk=512), "locality"),
    # three head groups per block (workgroups numbered (xcd, group, block))
    "h48_topk": (small_variant(PREFILL, mla_heads=48, topk=160), "topk"),
    # positions past one 32K-position membership window of the union kernel
    "h64_topk_L70000": (small_variant(PREFILL, batch=1, lens=(70000,), q_per_seq=(6,), topk=512),
                        "topk"),
    "h8_locality_L70000": (small_variant(PREFILL, batch=1, lens=(70000,), q_per_seq=(11,),
                                         mla_heads=8, topk=300), "locality"),
    # page size 4: windows of 2048 pages (8192 positions), the staged page slice full
    "h16_topk_P4_L20000": (small_variant(PREFILL, batch=1, lens=(20000,), q_per_seq=(5,),
                                         mla_heads=16, page_size=4, topk=256), "topk"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_qblocked_matches_oracle(name, dev):
    wl, sel = CASES[name]
    print(f"[qblock] {name}", flush=True)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    if sel == "topk":
        _, idx, _ = P.run_gpu(inp)
    else:
        idx = locality_indices(inp_h.seq_lens_host, inp_h.q_lens_host, wl.topk, wl.page_size,
                               block=8, hot_pages=max(2, wl.topk // wl.page_size + 2),
                               seed=3).to(dev)
        P.check_invariants(inp, idx, wl.topk)
    _check(inp, inp_h, idx)


def test_qblocked_fallback_on_caller_lists(dev):
    """Repeats, -1, positions past t and unsorted entries (the rows' lists are not
    mergeable): every entry is attended as given; the oracle sees the list with the
    out-of-range entries set to -1 and repeats kept."""
    wl = small_variant(PREFILL, topk=256)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    _, pos = O.row_positions(inp_h.seq_lens_host, inp_h.q_lens_host)
    g = np.random.default_rng(5)
    raw = g.integers(-3, max(inp_h.seq_lens_host) + 40, size=(inp.total_q, wl.topk)).astype(np.int32)
    raw[g.random(raw.shape) < 0.1] = raw[0, 0]
    raw[g.random(raw.shape) < 0.05] = -1
    masked = np.where((raw >= 0) & (raw <= pos[:, None]), raw, -1).astype(np.int32)
    _check(inp, inp_h, torch.from_numpy(raw).to(dev), torch.from_numpy(masked))
    # sorted lists except one row of a block: only that block falls back
    srt = np.sort(np.where(masked >= 0, masked, np.iinfo(np.int32).max), axis=1)
    srt = np.where(srt == np.iinfo(np.int32).max, -1, srt).astype(np.int32)
    for r in range(srt.shape[0]):  # distinct valid entries, ascending, -1 after
        v = np.unique(srt[r][srt[r] >= 0])
        srt[r] = -1
        srt[r, : v.size] = v
    srt[1, :2] = srt[1, :2][::-1].copy()
    _check(inp, inp_h, torch.from_numpy(srt).to(dev))


def test_qblocked_decode_batch_spans_sequences(dev):
    """One query per sequence: a block's rows are in different sequences, so the
    unions are concatenations; the result is still the per-query attention."""
    wl = small_variant("decode_b32_l8k", batch=6, lens=(700, 1300, 90, 2000, 64, 333), topk=128)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    _, idx, _ = P.run_gpu(inp)
    _check(inp, inp_h, idx)


def test_qblocked_rows_without_entries(dev):
    """Blocks whose rows list nothing (all -1) give an empty union (output 0, lse
    -inf), on the merge path and on the fallback; a fallback block where only
    some rows have entries reads its unused slots from a written row, so the
    poisoned pages of the pool never reach the sums."""
    wl = small_variant("decode_b32_l8k", batch=6, lens=(700, 1300, 90, 2000, 64, 333), topk=128)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    _, idx, _ = P.run_gpu(inp)
    idx = idx.clone()
    idx[0:4] = -1  # block 0: rows of four sequences, nothing listed
    idx[4] = -1    # block 1: only row 5 has entries
    _check(inp, inp_h, idx)
    inp_h = make_inputs(PREFILL)
    inp = to_device(inp_h, dev)
    _, idx, _ = P.run_gpu(inp)
    idx = idx.clone()
    idx[4:8] = -1  # a block of one sequence, nothing listed: merge path
    _check(inp, inp_h, idx)


def test_qblocked_union_over_several_chunks(dev):
    """Eight-query blocks (8 heads) whose selections barely overlap: unions of up to
    8 x 2048 slots, walked in row-table chunks of 2048."""
    wl = small_variant("prefill_q4k_l32k", batch=1, lens=(9000,), q_per_seq=(19,), mla_heads=8,
                       topk=2048, page_size=128)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    _, idx, _ = P.run_gpu(inp)
    _check(inp, inp_h, idx)


def test_qblocked_restart_on_late_large_logits(dev):
    """Rows 64..95 of the sequence scaled by 100: their logits exceed the reference
    fixed by the union's first tile by far more than the headroom, so the union is
    walked again from raised references."""
    wl = small_variant(PREFILL, batch=1, lens=(600,), q_per_seq=(9,), topk=1024)
    inp_h = make_inputs(wl)
    ps = wl.page_size
    cache = inp_h.kv_cache[0]
    for p_ in range(64, 96):
        page = int(inp_h.block_table[0, p_ // ps])
        cache[page, p_ % ps] = (cache[page, p_ % ps].float() * 100.0).to(cache.dtype)
    inp = to_device(inp_h, dev)
    _, idx, _ = P.run_gpu(inp)
    out, lse, _, _ = _run(inp, idx)
    assert torch.isfinite(out).all()
    P.check_mla(inp, 0, idx, out, lse, list(range(inp.total_q)), host_view(inp_h))


def test_qblocked_rejects_unsupported(dev):
    wl = small_variant(PREFILL, mla_heads=12, topk=64)
    inp = to_device(make_inputs(wl), dev)
    idx = torch.zeros((inp.total_q, 64), dtype=torch.int32, device=dev)
    with pytest.raises(dsa.DSAError):  # 12 heads: neither 8 nor a multiple of 16
        dsa.sparse_mla_fwd_qblocked(P.batch_of(inp), inp.q_mla[0], dsa.PagedCache(inp.kv_cache[0]),
                                    idx, wl.d_latent, wl.scale)


def test_qblocked_without_lse_and_empty_batch(dev):
    """lse may be left out (out unchanged bit for bit); an empty batch is a no-op."""
    inp_h = make_inputs(PREFILL)
    inp = to_device(inp_h, dev)
    _, idx, _ = P.run_gpu(inp)
    wl = inp.wl
    b = P.batch_of(inp)
    kv = dsa.PagedCache(inp.kv_cache[0])
    o1, l1 = dsa.sparse_mla_fwd_qblocked(b, inp.q_mla[0], kv, idx, wl.d_latent, wl.scale)
    o2, l2 = dsa.sparse_mla_fwd_qblocked(b, inp.q_mla[0], kv, idx, wl.d_latent, wl.scale,
                                         want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2)
    # sequences with no query row this step: total_q = 0
    empty = dsa.Batch(inp.block_table, inp.seq_lens, torch.zeros_like(inp.cu_q), 0,
                      inp.max_seq_len, 0)
    q0 = inp.q_mla[0][:0]
    o3, l3 = dsa.sparse_mla_fwd_qblocked(empty, q0, kv, idx[:0], wl.d_latent, wl.scale)
    torch.cuda.synchronize()
    assert o3.shape[0] == 0 and l3.shape[0] == 0
