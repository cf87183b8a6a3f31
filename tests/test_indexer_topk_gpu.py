"""GPU parity of dsa_indexer_topk, the indexer with the top-k fused into its
launch ("Making GLM-5.2 Sparse on TPUs", section "Stream indexer scores over
live context").

The fused call must return what dsa_indexer_scores followed by dsa_topk
return, bit for bit: the same score at every legal position and the same
indices (on identical scores the selection is exact and its result unique).
The indices are also checked against the oracle's top-k of the GPU's own
scores (bit-exact) and, end to end, against the oracle's top-k of the
oracle's scores inside the 1e-3 band; the scores against the oracle at the
1e-2 RMS bar. The per-row state must be zero-filled again after every call,
and nothing may be written past the outputs.
"""

import pytest
import torch

from tests import parity as P
from workloads import host_view, make_inputs, small_variant, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0x7EADBEEF

CASES = {
    # rows above, at, one past and below k, and a row of one position
    "bf16_ragged_k2048": small_variant("decode_b32_l8k", batch=6,
                                       lens=(8192, 5000, 2049, 2048, 300, 1), topk=2048),
    "fp8_keys": small_variant("indexshare_b64", batch=4, lens=(8000, 3000, 700, 64), topk=512,
                              n_layers=1),
    "h16_page128": small_variant("decode_b32_l8k", batch=3, lens=(7000, 1000, 129), idx_heads=16,
                                 page_size=128, topk=256),
    "h64_k300": small_variant("decode_b32_l8k", batch=3, lens=(4000, 1500, 90), idx_heads=64,
                              topk=300),
    # rows past 8K: 64 candidates per lane in the final selection
    "rows_16k": small_variant("decode_b32_l8k", batch=3, lens=(16384, 9000, 8193), topk=2048),
    # k of one and an odd k, 16 heads on fp8 keys
    "fp8_h16_k1": small_variant("indexshare_b64", batch=3, lens=(5000, 64, 1), idx_heads=16,
                                topk=1, n_layers=1),
    "bf16_k17": small_variant("decode_b32_l8k", batch=3, lens=(3000, 17, 16), topk=17),
    # a sequence without a query row between two with one
    "seq_without_row": small_variant("decode_b32_l8k", batch=3, lens=(700, 300, 65),
                                     q_per_seq=(1, 0, 1), topk=128),
}


def _dsa():
    import sparse_attention_decode_lightning_amd as dsa
    return dsa


def _two_call(dsa, inp, k):
    T, ld = inp.total_q, max(1, inp.max_seq_len)
    dev = inp.q_idx.device
    s = torch.full((T, ld), float("nan"), dtype=torch.float32, device=dev)
    i = torch.full((T, k), SENTINEL, dtype=torch.int32, device=dev)
    b = P.batch_of(inp)
    dsa.indexer_scores(b, inp.q_idx, inp.w, P.keys_of(inp), scores=s)
    dsa.topk(b, s, k, indices=i)
    return s, i


def _fused(dsa, inp, k, state=None):
    """The fused call with a guard row past scores and indices and 256 guard
    bytes past the state; returns (scores, indices, state)."""
    T, ld = inp.total_q, max(1, inp.max_seq_len)
    dev = inp.q_idx.device
    s = torch.full((T + 1, ld), float("nan"), dtype=torch.float32, device=dev)
    i = torch.full((T + 1, k), SENTINEL, dtype=torch.int32, device=dev)
    need = dsa.indexer_topk_state_size(T)
    if state is None:
        state = torch.zeros(need + 256, dtype=torch.uint8, device=dev)
    dsa.indexer_topk(P.batch_of(inp), inp.q_idx, inp.w, P.keys_of(inp), k, scores=s[:T],
                     indices=i[:T], state=state[:need])
    torch.cuda.synchronize()
    assert torch.isnan(s[T]).all(), "write past the scores buffer"
    assert (i[T] == SENTINEL).all(), "write past the indices buffer"
    assert int(state.count_nonzero()) == 0, "state not zero-filled after the call"
    return s[:T], i[:T], state


def _assert_same(inp, s1, i1, s2, i2):
    _, pos = P.positions(inp)
    for r in range(inp.total_q):
        t = int(pos[r])
        assert torch.equal(s1[r, : t + 1], s2[r, : t + 1]), f"row {r}: scores differ"
        assert torch.isnan(s1[r, t + 1:]).all(), f"row {r}: wrote past its causal bound"
    assert torch.equal(i1, i2), "indices differ from the two-call route"


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_two_calls_and_oracle(name):
    dsa = _dsa()
    wl = CASES[name]
    inp_h = make_inputs(wl)
    inp = to_device(inp_h, torch.device("cuda:0"))
    k = wl.topk
    s2, i2 = _two_call(dsa, inp, k)
    s1, i1, _ = _fused(dsa, inp, k)
    _assert_same(inp, s1, i1, s2, i2)
    rows = list(range(inp.total_q))
    P.check_invariants(inp, i1, k)
    P.check_topk_identical(s1, i1, rows, inp, k)
    host = host_view(inp_h)
    ref = P.check_scores(inp, s1, rows, host)
    P.check_topk_band(ref, i1, rows, k)


def test_state_reused_by_a_smaller_batch():
    """One state buffer, two calls in a row, the second with fewer rows and
    shorter sequences: each matches its two-call result, and the state is
    zero after each."""
    dsa = _dsa()
    dev = torch.device("cuda:0")
    big = to_device(make_inputs(CASES["bf16_ragged_k2048"]), dev)
    small = to_device(make_inputs(small_variant("decode_b32_l8k", batch=2, lens=(3000, 2500),
                                                topk=2048, seed=11)), dev)
    _, _, state = _fused(dsa, big, 2048)
    for inp in (big, small):
        s2, i2 = _two_call(dsa, inp, 2048)
        s1, i1, state = _fused(dsa, inp, 2048, state=state)
        _assert_same(inp, s1, i1, s2, i2)


def test_all_equal_scores_keep_the_lowest_positions():
    """Zero queries make every score 0: each row keeps positions 0 .. k-1 (the
    tie rule), through the row histogram's single bin."""
    dsa = _dsa()
    inp = to_device(make_inputs(small_variant("decode_b32_l8k", batch=3, lens=(6000, 2100, 50),
                                              topk=2048)), torch.device("cuda:0"))
    inp.q_idx.zero_()
    s2, i2 = _two_call(dsa, inp, 2048)
    s1, i1, _ = _fused(dsa, inp, 2048)
    _assert_same(inp, s1, i1, s2, i2)
    want = torch.arange(2048, dtype=torch.int32, device=i1.device)
    assert torch.equal(i1[0], want) and torch.equal(i1[1], want)
    assert torch.equal(i1[2, :50], want[:50]) and (i1[2, 50:] == -1).all()


def test_full_decode_batch_every_row():
    """The 32 x 8,192 decode batch: every row identical to the two-call route."""
    dsa = _dsa()
    from workloads import WORKLOADS
    wl = WORKLOADS["decode_b32_l8k"]
    inp = to_device(make_inputs(wl), torch.device("cuda:0"))
    s2, i2 = _two_call(dsa, inp, wl.topk)
    s1, i1, _ = _fused(dsa, inp, wl.topk)
    _assert_same(inp, s1, i1, s2, i2)
    P.check_topk_identical(s1, i1, list(range(0, inp.total_q, 4)), inp, wl.topk)


def test_several_queries_per_sequence_are_unsupported():
    dsa = _dsa()
    inp = to_device(make_inputs(small_variant("verify_b8_l240k", batch=2, lens=(1500, 777),
                                              topk=256)), torch.device("cuda:0"))
    with pytest.raises(dsa.DSAError) as e:
        dsa.indexer_topk(P.batch_of(inp), inp.q_idx, inp.w, P.keys_of(inp), 256)
    assert e.value.code == 5  # DSA_ERR_UNSUPPORTED


def test_graph_replays_match_the_eager_call():
    """The state clears itself inside the kernel (no memset node), so a captured
    call replays correctly: three replays with eager calls between them, each
    equal to the eager result, and the state zero after each."""
    dsa = _dsa()
    inp = to_device(make_inputs(small_variant("decode_b32_l8k", batch=4,
                                              lens=(8192, 3000, 2049, 700), topk=2048)),
                    torch.device("cuda:0"))
    k = 2048
    s_ref, i_ref, _ = _fused(dsa, inp, k)
    T, ld = inp.total_q, inp.max_seq_len
    dev = inp.q_idx.device
    s = torch.zeros((T, ld), dtype=torch.float32, device=dev)
    i = torch.zeros((T, k), dtype=torch.int32, device=dev)
    state = torch.zeros(dsa.indexer_topk_state_size(T), dtype=torch.uint8, device=dev)
    b, keys = P.batch_of(inp), P.keys_of(inp)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm the call on the capture stream
        dsa.indexer_topk(b, inp.q_idx, inp.w, keys, k, scores=s, indices=i, state=state)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsa.indexer_topk(b, inp.q_idx, inp.w, keys, k, scores=s, indices=i, state=state)
    torch.cuda.synchronize()
    for _ in range(3):
        i.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(i, i_ref), "graph replay differs from the eager call"
        assert int(state.count_nonzero()) == 0, "state not zero-filled after a replay"
        _fused(dsa, inp, k)  # eager work between replays
