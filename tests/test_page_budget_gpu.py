"""GPU parity of page-budget selection (dsa_page_scores, dsa_page_topk,
dsa_indexer_page_scores) against the oracle.

Page maxima are compared bit-exact on the GPU's own token scores, with the
score buffer past each row's causal bound filled with huge values (a page's
maximum must never see them); the page top-k and its token expansion are
compared bit-exact on the GPU's own page scores; attention over the expanded
positions within the 1e-2 RMS bar. The page maxima that the indexer pools on
chip are compared with the oracle's page maxima of the oracle's float64
scores (the scores' 1e-2 RMS bar: a maximum moves by at most the largest
error of the scores it ranges over), and end to end the GPU's kept pages may
differ from the oracle's only where the oracle page score lies within
1e-3 |kp-th oracle page score| of the kp-th one. Pages of one position must reproduce the
token top-k exactly, on a row long enough for the two-phase selection.
"""

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from tests import parity as P
from workloads import host_view, make_inputs, small_variant, to_device

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_decode_lightning_amd as dsa
    return dsa


def _scores_with_poison(inp, dsa, b):
    T, ld = inp.total_q, max(1, inp.max_seq_len)
    scores = torch.full((T, ld), 3.0e38, dtype=torch.float32, device=inp.q_idx.device)
    dsa.indexer_scores(b, inp.q_idx, inp.w, P.keys_of(inp), scores=scores)
    return scores


CASES = [
    # (base workload, overrides, page size, page budget)
    # the 4,096-token prefill budget of 32 pages of 128 ("Making GLM-5.2 Sparse on TPUs",
    # section "Separate the indexer from the attention it controls"): k = 4096 in the MLA
    ("decode_b32_l8k", dict(batch=2, lens=(6000, 4500), topk=256, page_size=128), 128, 32),
    ("decode_b32_l8k", dict(batch=3, lens=(1500, 700, 64), topk=256), 64, 8),
    ("verify_b8_l240k", dict(batch=2, lens=(3000, 1100), topk=256), 64, 5),
    ("decode_b32_l8k", dict(batch=2, lens=(2000, 513), topk=256, page_size=16), 16, 20),
    ("tiny", dict(), 16, 3),
]


@pytest.mark.parametrize("base,kw,page,kp", CASES, ids=[f"{c[0]}-P{c[2]}-kp{c[3]}" for c in CASES])
def test_page_budget_matches_oracle(base, kw, page, kp):
    dsa = _dsa()
    wl = small_variant(base, **kw)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, torch.device("cuda:0"))
    host = host_view(inp_h)
    b = P.batch_of(inp)
    scores = _scores_with_poison(inp, dsa, b)
    n_pages = -(-inp.max_seq_len // page)
    ps = torch.full((inp.total_q + 1, n_pages), float("nan"), dtype=torch.float32,
                    device=scores.device)
    dsa.page_scores(b, scores, page, out=ps[: inp.total_q])
    pages, idx = dsa.page_topk(b, ps[: inp.total_q], page, kp)
    torch.cuda.synchronize()
    assert torch.isnan(ps[inp.total_q]).all(), "write past the page scores"
    _, pos = P.positions(inp)
    s = scores.double().cpu().numpy()
    g_ps = ps[: inp.total_q].double().cpu().numpy()
    g_pages = pages.cpu().numpy()
    g_idx = idx.cpu().numpy()
    for r in range(inp.total_q):
        t = int(pos[r])
        ref_ps = O.page_scores_row(s[r, : t + 1], page)
        n = len(ref_ps)
        assert np.array_equal(g_ps[r, :n], ref_ps), f"row {r}: page maxima differ"
        assert np.isnan(g_ps[r, n:]).all(), f"row {r}: wrote a page past t"
        ref_pages = O.topk_row(g_ps[r, :n], kp)
        assert np.array_equal(g_pages[r], ref_pages), f"row {r}: page top-k differs"
        assert np.array_equal(g_idx[r], O.expand_pages(ref_pages, page, t)), f"row {r}: expansion"
    # attention over the expanded positions
    out, lse = dsa.sparse_mla_fwd(b, inp.q_mla[0], dsa.PagedCache(inp.kv_cache[0]), idx,
                                  wl.d_latent, wl.scale)
    torch.cuda.synchronize()
    P.check_mla(inp, 0, idx, out, lse, list(range(inp.total_q)), host)


def test_unit_pages_reproduce_token_topk_on_long_rows():
    """Pages of one position: dsa_page_topk == dsa_topk, on rows long enough (40,000
    positions) for the two-phase selection."""
    dsa = _dsa()
    wl = small_variant("verify_b8_l240k", batch=2, lens=(40000, 35001), q_per_seq=2, topk=2048,
                       page_size=64)
    inp = to_device(make_inputs(wl), torch.device("cuda:0"))
    b = P.batch_of(inp)
    scores = _scores_with_poison(inp, dsa, b)
    ps = dsa.page_scores(b, scores, 1)
    pages, idx = dsa.page_topk(b, ps, 1, wl.topk)
    tok = dsa.topk(b, scores, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(pages, tok) and torch.equal(idx, tok)


def test_page_topk_rejects_bad_arguments():
    dsa = _dsa()
    wl = small_variant("tiny")
    inp = to_device(make_inputs(wl), torch.device("cuda:0"))
    b = P.batch_of(inp)
    ps = torch.zeros((inp.total_q, 16), dtype=torch.float32, device=inp.q_idx.device)
    with pytest.raises(dsa.DSAError):
        dsa.page_topk(b, ps, 16, 0)
    with pytest.raises(dsa.DSAError):  # ld_pages shorter than ceil(max_seq_len / page)
        dsa.page_topk(b, ps[:, :3], 16, 2)


FUSED = [
    # (base workload, overrides, selection page size)
    ("decode_b32_l8k", dict(batch=3, lens=(1500, 700, 64), topk=256), 64),
    ("decode_b32_l8k", dict(batch=3, lens=(5000, 1025, 130), topk=256), 64),
    ("verify_b8_l240k", dict(batch=2, lens=(3000, 1100), topk=256), 64),
    ("verify_b8_l240k", dict(batch=3, lens=(4100, 2049, 65), topk=256), 64),
    ("decode_b32_l8k", dict(batch=2, lens=(900, 333), topk=256, idx_heads=64,
                            w_std=0.125), 64),
    ("decode_b32_l8k", dict(batch=2, lens=(1900, 333), topk=256, idx_heads=16,
                            w_std=0.25, page_size=128), 64),
]


@pytest.mark.parametrize("base,kw,page", FUSED, ids=[f"{c[0]}-P{c[2]}" for c in FUSED])
def test_fused_page_scores_equal_two_call_route(base, kw, page):
    """dsa_indexer_page_scores writes exactly what dsa_indexer_scores + dsa_page_scores
    write (same per-token arithmetic), and nothing past each row's last legal page."""
    dsa = _dsa()
    wl = small_variant(base, **kw)
    inp = to_device(make_inputs(wl), torch.device("cuda:0"))
    b = P.batch_of(inp)
    n_pages = -(-inp.max_seq_len // page)
    scores = _scores_with_poison(inp, dsa, b)
    two = torch.full((inp.total_q, n_pages), float("nan"), device=scores.device)
    dsa.page_scores(b, scores, page, out=two)
    fused = torch.full((inp.total_q + 1, n_pages + 3), float("nan"), device=scores.device)
    dsa.indexer_page_scores(b, inp.q_idx, inp.w, P.keys_of(inp), page,
                            out=fused[: inp.total_q])
    torch.cuda.synchronize()
    assert torch.isnan(fused[inp.total_q]).all() and torch.isnan(fused[:, n_pages:]).all()
    a, c = fused[: inp.total_q, :n_pages].cpu().numpy(), two.cpu().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(c))
    assert np.array_equal(a[~np.isnan(a)].view(np.uint32), c[~np.isnan(c)].view(np.uint32))


def test_fused_page_scores_unsupported_shapes():
    dsa = _dsa()
    wl = small_variant("decode_b32_l8k", batch=1, lens=(500,), topk=256)
    inp = to_device(make_inputs(wl), torch.device("cuda:0"))
    b = P.batch_of(inp)
    for page in (16, 128, 1024):  # only pages of one streamed 64-key block
        with pytest.raises(dsa.DSAError):
            dsa.indexer_page_scores(b, inp.q_idx, inp.w, P.keys_of(inp), page)


def _page_band(ref_ps: np.ndarray, gpu_pages: np.ndarray, kp: int, where: str):
    """Kept page sets (GPU vs oracle on the oracle's scores) differ only inside the band."""
    ref = O.topk_row(ref_ps, kp)
    a = set(int(x) for x in ref if x >= 0)
    b = set(int(x) for x in gpu_pages if x >= 0)
    assert len(a) == len(b), where
    if a == b:
        return 0
    kth = np.sort(ref_ps)[::-1][min(kp, len(ref_ps)) - 1]
    for p in a ^ b:
        assert abs(ref_ps[p] - kth) <= P.BAND * abs(kth), (where, p, ref_ps[p], kth)
    return len(a ^ b)


@pytest.mark.parametrize("base,kw,page", FUSED, ids=[f"{c[0]}-P{c[2]}" for c in FUSED])
def test_fused_page_scores_match_oracle(base, kw, page):
    """dsa_indexer_page_scores against the oracle's page maxima of its own float64 scores,
    within the indexer's 1e-2 RMS bar, and nothing written past a row's last legal page."""
    dsa = _dsa()
    wl = small_variant(base, **kw)
    print(f"[fused-page-oracle] {base} {kw}", flush=True)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, torch.device("cuda:0"))
    host = host_view(inp_h)
    b = P.batch_of(inp)
    n_pages = -(-inp.max_seq_len // page)
    fused = torch.full((inp.total_q, n_pages), float("nan"), device=inp.q_idx.device)
    dsa.indexer_page_scores(b, inp.q_idx, inp.w, P.keys_of(inp), page, out=fused)
    torch.cuda.synchronize()
    ref = O.indexer_scores(host)
    rms = np.sqrt(np.mean(np.concatenate([v for v in ref.values()]) ** 2))
    got = fused.double().cpu().numpy()
    worst = 0.0
    for r in range(inp.total_q):
        ref_ps = O.page_scores_row(ref[r], page)
        n = len(ref_ps)
        assert np.isfinite(got[r, :n]).all(), f"row {r}: non-finite page score"
        assert np.isnan(got[r, n:]).all(), f"row {r}: wrote a page past t"
        worst = max(worst, float(np.max(np.abs(got[r, :n] - ref_ps))))
    assert worst <= P.SCORE_TOL * rms, (worst, rms)


BAND_CASES = CASES + [("decode_b32_l8k", dict(batch=4, lens=(8192, 3000, 900, 64), topk=256), 64, 32)]


@pytest.mark.parametrize("base,kw,page,kp", BAND_CASES,
                         ids=[f"{c[0]}-P{c[2]}-kp{c[3]}" for c in BAND_CASES])
def test_page_budget_end_to_end_band(base, kw, page, kp):
    """GPU pages from GPU scores against oracle pages from oracle scores: they may differ
    only inside the 1e-3 band around the kp-th oracle page score, on the two-call route
    and, where the indexer pools page maxima itself, on the fused route."""
    dsa = _dsa()
    wl = small_variant(base, **kw)
    print(f"[page-band] {base} {kw} P={page} kp={kp}", flush=True)
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, torch.device("cuda:0"))
    host = host_view(inp_h)
    b = P.batch_of(inp)
    scores = _scores_with_poison(inp, dsa, b)
    routes = {"two-call": dsa.page_scores(b, scores, page)}
    try:
        routes["fused"] = dsa.indexer_page_scores(b, inp.q_idx, inp.w, P.keys_of(inp), page)
    except dsa.DSAError:
        pass
    ref = O.indexer_scores(host)
    _, pos = P.positions(inp)
    differ = 0
    for name, ps in routes.items():
        pages, idx = dsa.page_topk(b, ps, page, kp)
        torch.cuda.synchronize()
        g_pages, g_idx = pages.cpu().numpy(), idx.cpu().numpy()
        for r in range(inp.total_q):
            t = int(pos[r])
            differ += _page_band(O.page_scores_row(ref[r], page), g_pages[r], kp, f"{name} row {r}")
            assert np.array_equal(g_idx[r], O.expand_pages(g_pages[r], page, t)), (name, r)
    print(f"[page-band] pages differing inside the band: {differ}", flush=True)
