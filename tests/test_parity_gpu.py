"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Small cases are compared element by element (several tiles and ragged tails,
every kernel variant); the full-size workloads run in the launch
configuration the benchmark times and are compared on every row (every 64th
row of the 4,096-row prefill chunk), with the index invariants checked on
every row.
"""

import numpy as np
import pytest
import torch

import sparse_attention_decode_lightning_amd as dsa
from tests import parity as P
from workloads import WORKLOADS, host_view, make_inputs, small_variant, to_device

pytestmark = pytest.mark.gpu

BF16_DECODE = small_variant("decode_b32_l8k", batch=3, lens=(300, 1000, 2071), topk=256)
SMALL_CASES = {
    "tiny_f32": WORKLOADS["tiny"],
    "bf16_decode_ragged": BF16_DECODE,
    "fp8_decode_ragged": small_variant("indexshare_b64", batch=4, lens=(2049, 100, 777, 4096),
                                       topk=512, n_layers=2),
    "fp8_multiquery": small_variant("verify_b8_l240k", batch=2, lens=(1500, 777), topk=256),
    "bf16_prefill": small_variant("prefill_q4k_l32k", batch=1, lens=1200, q_per_seq=300,
                                  topk=256),
    # prefill kernel: 64 heads, ragged query counts (some below one query
    # block, one equal to its sequence), pages of 48 across 64-key blocks
    "bf16_prefill_h64_ragged": small_variant("prefill_q4k_l32k", batch=3, lens=(900, 257, 70),
                                             q_per_seq=(40, 17, 70), idx_heads=64,
                                             page_size=48, topk=128),
    # prefill kernel, 128-key blocks: 32 heads on pages of 64 (two pages per
    # block), and 64 heads on pages of 128 (one page per block); ragged tails
    "bf16_prefill_p64": small_variant("prefill_q4k_l32k", batch=2, lens=(1000, 130),
                                      q_per_seq=(40, 16), page_size=64, topk=128),
    "bf16_prefill_h64_p128": small_variant("prefill_q4k_l32k", batch=2, lens=(700, 300),
                                           q_per_seq=(20, 17), idx_heads=64, topk=128),
    # whole key blocks per page on the other block sizes: 16 heads (64-key
    # blocks) on pages of 64, 32 heads on pages of 256 (two blocks per page)
    "bf16_prefill_h16_p64": small_variant("prefill_q4k_l32k", batch=2, lens=(700, 200),
                                          q_per_seq=(40, 16), idx_heads=16, page_size=64,
                                          topk=64),
    "bf16_prefill_p256": small_variant("prefill_q4k_l32k", batch=2, lens=(1100, 300),
                                       q_per_seq=(33, 20), page_size=256, topk=128),
    # prefill kernel: 16 heads (32 rows per workgroup), pages of 16
    "bf16_prefill_h16": small_variant("prefill_q4k_l32k", batch=2, lens=(500, 333),
                                      q_per_seq=(33, 20), idx_heads=16, page_size=16, topk=64),
    "edge_lengths": small_variant(BF16_DECODE, batch=4, lens=(5, 1, 70, 64), q_per_seq=(1, 0, 3, 1),
                                  topk=64),
    "page_size_1": small_variant(BF16_DECODE, batch=2, lens=(130, 47), page_size=1, topk=32),
    "page_size_16_k_ge_len": small_variant(BF16_DECODE, batch=2, lens=(200, 333), page_size=16,
                                           topk=512),
    "idx64_heads": small_variant(BF16_DECODE, batch=2, lens=(500, 260), idx_heads=64, topk=128),
    "idx16_heads_multiq": small_variant("verify_b8_l240k", batch=2, lens=(400, 90), q_per_seq=5,
                                        idx_heads=16, topk=64),
    # four query rows of 32 heads with bf16 keys (the 32x32 MFMA path of the
    # streaming indexer), one group short of four rows, one sequence shorter
    # than a block
    "bf16_multiquery_h32": small_variant(BF16_DECODE, batch=3, lens=(700, 300, 40),
                                         q_per_seq=(4, 3, 4), topk=128),
    "topk_two_phase": small_variant("indexshare_b64", batch=4, lens=(70000, 33000, 5000, 300),
                                    topk=512, n_layers=1),
    "mla_generic_bf16": small_variant(BF16_DECODE, batch=2, lens=(300, 129), mla_heads=16,
                                      d_latent=128, d_rope=32, topk=100),
    # 64-head MFMA MLA with k not a multiple of the 32-row tile: one split
    # ending in a partial tile (k = 100), a single partial tile (k = 17), and
    # many splits whose last one is one row short (k = 2047)
    "mla_mfma_k100": small_variant(BF16_DECODE, batch=3, lens=(300, 1000, 77), topk=100),
    "mla_mfma_k17": small_variant(BF16_DECODE, batch=3, lens=(300, 1000, 9), topk=17),
    "mla_mfma_k2047": small_variant(BF16_DECODE, batch=2, lens=(3000, 2071), q_per_seq=(2, 1),
                                    topk=2047),
    # the MFMA MLA with fewer than 64 heads (zero-query columns): 8 heads over
    # many splits, 40 heads (not a multiple of a wave's 16), 1 head with a
    # partial tile
    "mla_mfma_h8": small_variant(BF16_DECODE, batch=3, lens=(3000, 700, 90), mla_heads=8,
                                 topk=1000),
    "mla_mfma_h40": small_variant(BF16_DECODE, batch=2, lens=(900, 300), q_per_seq=(3, 1),
                                  mla_heads=40, topk=200),
    "mla_mfma_h1_k17": small_variant(BF16_DECODE, batch=2, lens=(300, 64), mla_heads=1,
                                     topk=17),
}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_small_case_full_parity(name, dev):
    wl = SMALL_CASES[name]
    print(f"[parity] {name}", flush=True)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    host = host_view(inp_h)
    scores, idx, outs = P.run_gpu(inp)
    rows = list(range(inp.total_q))
    ref_scores = P.check_scores(inp, scores, rows, host)
    P.check_topk_identical(scores, idx, rows, inp, wl.topk)
    P.check_topk_band(ref_scores, idx, rows, wl.topk)
    P.check_invariants(inp, idx, wl.topk)
    for l, (out, lse) in enumerate(outs):
        P.check_mla(inp, l, idx, out, lse, rows, host)


def test_indexshare_layers_reuse_one_topk(dev):
    """One top-k buffer serves several layers; each layer's output is its own oracle's."""
    wl = small_variant("indexshare_b64", batch=3, lens=(3000, 2100, 5000), topk=1024, n_layers=3)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    _, idx, outs = P.run_gpu(inp)
    host = host_view(inp_h)
    rows = list(range(inp.total_q))
    for l, (out, lse) in enumerate(outs):
        P.check_mla(inp, l, idx, out, lse, rows, host)
    assert not torch.equal(outs[0][0], outs[1][0])


@pytest.mark.parametrize("name,n_layers,heads", [("indexshare_b64", 3, 64),
                                                  ("indexshare_b64", 2, 24), ("tiny", 2, 8)])
def test_mla_layers_call_equals_one_call_per_layer(name, n_layers, heads, dev):
    """IndexShare as one call over several layers is bit-identical to one call per
    layer (MFMA path with splits, also with 24 heads; generic path), canaries past
    every output intact, and lse may be left out."""
    wl = small_variant(name, batch=3, lens=(3000, 2100, 5000) if name != "tiny" else (256, 90, 17),
                       topk=1024 if name != "tiny" else 64, n_layers=n_layers, mla_heads=heads)
    print(f"[mla-layers] {name} x{n_layers} h{heads}", flush=True)
    inp = to_device(make_inputs(wl), dev)
    _, idx, ref = P.run_gpu(inp)
    T = inp.total_q
    kvs = [dsa.PagedCache(inp.kv_cache[l]) for l in range(n_layers)]
    outs = [torch.full((T + 1, wl.mla_heads, wl.d_latent), float("nan"), device=dev)
            for _ in range(n_layers)]
    lses = [torch.full((T + 1, wl.mla_heads), float("nan"), device=dev) for _ in range(n_layers)]
    dsa.sparse_mla_fwd_layers(P.batch_of(inp), [inp.q_mla[l] for l in range(n_layers)], kvs, idx,
                              wl.d_latent, wl.scale, outs=[o[:T] for o in outs],
                              lses=[x[:T] for x in lses])
    o2, l2 = dsa.sparse_mla_fwd_layers(P.batch_of(inp), [inp.q_mla[l] for l in range(n_layers)],
                                       kvs, idx, wl.d_latent, wl.scale, want_lse=False)
    # lse for some layers only (a NULL entry in the lse array)
    some = [x[:T].clone().fill_(float("nan")) if l % 2 == 0 else None for l, x in enumerate(lses)]
    o3, l3 = dsa.sparse_mla_fwd_layers(P.batch_of(inp), [inp.q_mla[l] for l in range(n_layers)],
                                       kvs, idx, wl.d_latent, wl.scale, lses=some)
    torch.cuda.synchronize()
    assert l2 is None
    for l in range(n_layers):
        assert torch.equal(outs[l][:T], ref[l][0]) and torch.equal(lses[l][:T], ref[l][1]), l
        assert torch.equal(o2[l], ref[l][0]) and torch.equal(o3[l], ref[l][0]), l
        assert (l3[l] is None) if l % 2 else torch.equal(l3[l], ref[l][1]), l
        assert torch.isnan(outs[l][T]).all() and torch.isnan(lses[l][T]).all()


def test_mla_restart_on_late_large_logits(dev):
    """Rows 64..95 of sequence 0 are scaled by 100, so their logits exceed the softmax
    reference fixed by the split's first tile by far more than the 2^64 headroom: the
    split is walked a second time from a raised reference, and the result is still the
    oracle's. With k >= L every position is selected, so the scaled rows are in the
    first split of row 0 (slots 0..127, tiles of 32) behind two ordinary tiles."""
    wl = small_variant(BF16_DECODE, batch=2, lens=(600, 300), topk=1024)
    inp_h = make_inputs(wl)
    ps = wl.page_size
    cache = inp_h.kv_cache[0]
    for pos in range(64, 96):
        page = int(inp_h.block_table[0, pos // ps])
        cache[page, pos % ps] = (cache[page, pos % ps].float() * 100.0).to(cache.dtype)
    inp = to_device(inp_h, dev)
    host = host_view(inp_h)
    scores, idx, outs = P.run_gpu(inp)
    rows = list(range(inp.total_q))
    P.check_invariants(inp, idx, wl.topk)
    out, lse = outs[0]
    assert torch.isfinite(out).all()
    P.check_mla(inp, 0, idx, out, lse, rows, host)


def test_block_table_permutation_invariance(dev):
    """Same logical caches under two different physical page layouts give identical outputs."""
    wl = small_variant(BF16_DECODE, batch=2, lens=(700, 1300))
    a_h = make_inputs(wl)
    b_h = make_inputs(wl.replace(seed=wl.seed))  # same draw
    pool = a_h.k_cache.shape[0]
    perm = torch.randperm(pool, generator=torch.Generator().manual_seed(99))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(pool)
    b_h.block_table = inv[a_h.block_table.long()].to(torch.int32)
    b_h.k_cache = torch.empty_like(a_h.k_cache)
    b_h.k_cache[inv] = a_h.k_cache
    b_h.kv_cache = [torch.empty_like(c) for c in a_h.kv_cache]
    b_h.kv_cache[0][inv] = a_h.kv_cache[0]
    sa, ia, oa = P.run_gpu(to_device(a_h, dev))
    sb, ib, ob = P.run_gpu(to_device(b_h, dev))
    for r in range(a_h.total_q):
        t = a_h.seq_lens_host[r] - 1
        assert torch.equal(sa[r, : t + 1], sb[r, : t + 1])
    assert torch.equal(ia, ib)
    assert torch.equal(oa[0][0], ob[0][0])


def test_mutated_metadata_is_detected(dev):
    """Feeding a swapped block-table row must break parity (the comparison is sensitive)."""
    wl = small_variant(BF16_DECODE, batch=2, lens=(1024, 1024), topk=128)
    inp_h = make_inputs(wl)
    bad_h = make_inputs(wl)
    bad_h.block_table = bad_h.block_table.flip(0).contiguous()
    scores, _, _ = P.run_gpu(to_device(bad_h, dev))
    with pytest.raises(AssertionError):
        P.check_scores(inp_h, scores, [0, 1], host_view(inp_h))


FULL = ["decode_b32_l8k", "indexshare_b64", "prefill_q4k_l32k", "verify_b8_l240k"]
# every row of the decode-shaped workloads; every 64th row of the 4,096-row
# prefill chunk (its last row included)
SAMPLE_ROWS = {
    "decode_b32_l8k": list(range(32)),
    "indexshare_b64": list(range(64)),
    "prefill_q4k_l32k": list(range(0, 4096, 64)) + [4095],
    "verify_b8_l240k": list(range(32)),
}


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name, dev):
    wl = WORKLOADS[name]
    print(f"[parity-full] {name}", flush=True)
    inp = make_inputs(wl, device="cuda")
    scores, idx, outs = P.run_gpu(inp, canary=False)
    rows = SAMPLE_ROWS[name]
    host = host_view(inp, lazy=True)
    ref = P.check_scores(inp, scores, rows, host)
    P.check_topk_identical(scores, idx, rows, inp, wl.topk)
    P.check_topk_band(ref, idx, rows, wl.topk)
    P.check_invariants(inp, idx, wl.topk)
    for l, (out, lse) in enumerate(outs):
        assert torch.isfinite(out).all()
        P.check_mla(inp, l, idx, out, lse, rows, host)


def test_graph_replay_matches_eager(dev):
    """The three calls captured into a HIP graph replay bit-exactly, replay after replay,
    with unrelated eager work and synchronizations in between."""
    import sparse_attention_decode_lightning_amd as dsa

    wl = small_variant("indexshare_b64", batch=3, lens=(3000, 2100, 40000), topk=512, n_layers=2)
    inp = to_device(make_inputs(wl), dev)
    b, keys = P.batch_of(inp), P.keys_of(inp)
    T = inp.total_q
    scores = torch.zeros((T, inp.max_seq_len), dtype=torch.float32, device=dev)
    idx = torch.zeros((T, wl.topk), dtype=torch.int32, device=dev)
    outs = [torch.zeros((T, wl.mla_heads, wl.d_latent), dtype=torch.float32, device=dev)
            for _ in range(wl.n_layers)]
    tk_ws = torch.zeros(max(16, dsa.topk_workspace_size(T, inp.max_seq_len, wl.topk)),
                        dtype=torch.uint8, device=dev)
    ws = torch.zeros(max(16, dsa.sparse_mla_workspace_size(T, wl.mla_heads, wl.d_latent, wl.topk)),
                     dtype=torch.uint8, device=dev)

    def step():
        dsa.indexer_scores(b, inp.q_idx, inp.w, keys, scores=scores)
        dsa.topk(b, scores, wl.topk, indices=idx, workspace=tk_ws)
        for l in range(wl.n_layers):
            dsa.sparse_mla_fwd(b, inp.q_mla[l], dsa.PagedCache(inp.kv_cache[l]), idx, wl.d_latent,
                               wl.scale, out=outs[l], workspace=ws, want_lse=False)

    step()
    torch.cuda.synchronize()
    ref_idx, ref_out = idx.clone(), [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        idx.fill_(-7)
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {i}: indices differ"
        for o, r in zip(outs, ref_out):
            assert torch.equal(o, r), f"replay {i}: outputs differ"
        del junk


def _random_cases(n: int, seed: int):
    """Seeded random shapes across the dispatch space: page sizes that do and do not
    hold whole 64-key blocks, 16/32/64 indexer heads, bf16 and fp8 keys, query counts
    0..5 per sequence (some groups short of four), lengths from 1 to past 32K (the
    two-phase top-k), k from 64 to 2048."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(g.integers(1, 5))
        lens = tuple(int(x) for x in g.choice([1, 7, 64, 65, 300, 2049, 5000, 17000, 40000], size=B))
        qs = tuple(int(min(L, x)) for L, x in zip(lens, g.integers(0, 6, size=B)))
        if sum(qs) == 0:
            qs = (1,) + qs[1:]
        base = "indexshare_b64" if g.random() < 0.5 else "decode_b32_l8k"
        out.append((f"rand{i}", small_variant(
            base, seed=100 + i, batch=B, lens=lens, q_per_seq=qs,
            page_size=int(g.choice([16, 48, 64, 128])), idx_heads=int(g.choice([16, 32, 64])),
            topk=int(g.choice([64, 512, 2048])), n_layers=1)))
    return out


@pytest.mark.parametrize("name,wl", _random_cases(12, seed=7), ids=[c[0] for c in _random_cases(12, 7)])
def test_random_shapes_parity(name, wl, dev):
    """Scores within 1e-2 RMS, top-k identical on the GPU's scores and within the band
    end to end, index invariants, and MLA on a sample of rows, for random shapes."""
    print(f"[parity-rand] {name} lens={wl.lens} q={wl.q_per_seq} P={wl.page_size} "
          f"H={wl.idx_heads} k={wl.topk} keys={wl.idx_k_dtype}", flush=True)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, dev)
    host = host_view(inp_h)
    scores, idx, outs = P.run_gpu(inp)
    rows = sorted(set(np.random.default_rng(1).choice(inp.total_q, size=min(6, inp.total_q),
                                                      replace=False).tolist()))
    ref_scores = P.check_scores(inp, scores, rows, host)
    P.check_topk_identical(scores, idx, rows, inp, wl.topk)
    P.check_topk_band(ref_scores, idx, rows, wl.topk)
    P.check_invariants(inp, idx, wl.topk)
    out, lse = outs[0]
    P.check_mla(inp, 0, idx, out, lse, rows, host)
