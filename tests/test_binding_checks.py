"""The torch binding rejects inconsistent shapes on the host, before any pointer
reaches the C ABI (CPU only: the checks run before the device check, so CPU
tensors are enough to reach them).

The kernels size their work from the batch (sequence count, total_q), so a
batch whose arrays disagree with each other, or a per-row tensor or output
with fewer rows than total_q, would make them read or write past the caller's
buffers; the binding refuses both.
"""

import pytest
import torch

import sparse_attention_decode_lightning_amd as dsa

T, B, H, D, DL = 4, 2, 32, 128, 512


def _batch(total_q=T, B_=B, cu=None, bt_rows=None):
    cu = torch.tensor([0, 2, total_q], dtype=torch.int32) if cu is None else cu
    bt = torch.zeros((B_ if bt_rows is None else bt_rows, 8), dtype=torch.int32)
    return dsa.Batch(bt, torch.full((B_,), 300, dtype=torch.int32), cu, total_q, 300, 2)


def _keys():
    return dsa.PagedCache(torch.zeros((8, 64, D), dtype=torch.bfloat16))


def test_batch_arrays_must_agree():
    with pytest.raises(ValueError, match="cu_q must be"):
        _batch(cu=torch.tensor([0, 4], dtype=torch.int32)).c()
    with pytest.raises(ValueError, match="block_table must be"):
        _batch(bt_rows=3).c()
    # a consistent batch passes the shape checks and stops at the device check
    with pytest.raises(ValueError, match="on the GPU"):
        _batch().c()


def test_indexer_rows_must_cover_total_q():
    q = torch.zeros((T - 1, H, D), dtype=torch.bfloat16)
    w = torch.zeros((T - 1, H))
    with pytest.raises(ValueError, match="q_idx has 3 rows"):
        dsa.indexer_scores(_batch(), q, w, _keys())
    q = torch.zeros((T, H, D), dtype=torch.bfloat16)
    w = torch.zeros((T, H))
    with pytest.raises(ValueError, match="max_seq_len"):
        dsa.indexer_scores(_batch(), q, w, _keys(), scores=torch.zeros((T, 100)))
    with pytest.raises(ValueError, match="q_idx has 3 rows"):
        dsa.indexer_page_scores(_batch(), q[:3], w[:3], _keys(), 64)


def test_topk_rows_must_cover_total_q():
    with pytest.raises(ValueError, match="scores has 3 rows"):
        dsa.topk(_batch(), torch.zeros((T - 1, 300)), 64)
    with pytest.raises(ValueError, match="ld >= max_seq_len"):
        dsa.topk(_batch(), torch.zeros((T, 200)), 64)


def test_page_calls_check_rows_and_widths():
    with pytest.raises(ValueError, match="scores has 3 rows"):
        dsa.page_scores(_batch(), torch.zeros((T - 1, 300)), 64)
    with pytest.raises(ValueError, match="ld_pages"):
        dsa.page_scores(_batch(), torch.zeros((T, 300)), 64, out=torch.zeros((T, 4)))
    with pytest.raises(ValueError, match="page_scores has 3 rows"):
        dsa.page_topk(_batch(), torch.zeros((T - 1, 5)), 64, 2)


def test_mla_rows_and_outputs_are_checked():
    q = torch.zeros((T, 64, 576), dtype=torch.bfloat16)
    kv = dsa.PagedCache(torch.zeros((8, 64, 576), dtype=torch.bfloat16))
    idx = torch.zeros((T, 64), dtype=torch.int32)
    with pytest.raises(ValueError, match="q has 3 rows"):
        dsa.sparse_mla_fwd(_batch(), q[:3], kv, idx, DL, 0.0625)
    with pytest.raises(ValueError, match="indices has 3 rows"):
        dsa.sparse_mla_fwd(_batch(), q, kv, idx[:3], DL, 0.0625)
    with pytest.raises(ValueError, match="out must be"):
        dsa.sparse_mla_fwd(_batch(), q, kv, idx, DL, 0.0625, out=torch.zeros((T, 64, 256)))
    with pytest.raises(ValueError, match="out has 3 rows"):
        dsa.sparse_mla_fwd(_batch(), q, kv, idx, DL, 0.0625, out=torch.zeros((T - 1, 64, DL)))
    with pytest.raises(ValueError, match="lse must be"):
        dsa.sparse_mla_fwd(_batch(), q, kv, idx, DL, 0.0625, lse=torch.zeros((T, 32)))
    with pytest.raises(ValueError, match="out has 3 rows"):
        dsa.sparse_mla_fwd_layers(_batch(), [q, q], [kv, kv], idx, DL, 0.0625,
                                  outs=[torch.zeros((T, 64, DL)), torch.zeros((T - 1, 64, DL))])
    with pytest.raises(ValueError, match="lse must be"):
        dsa.sparse_mla_fwd_layers(_batch(), [q, q], [kv, kv], idx, DL, 0.0625,
                                  lses=[None, torch.zeros((T, 63))])


def test_indexer_topk_checks_rows_and_outputs():
    q = torch.zeros((T, H, D), dtype=torch.bfloat16)
    w = torch.zeros((T, H))
    with pytest.raises(ValueError, match="q_idx has 3 rows"):
        dsa.indexer_topk(_batch(), q[:3], w[:3], _keys(), 64)
    with pytest.raises(ValueError, match="w must be"):
        dsa.indexer_topk(_batch(), q, w[:, :16], _keys(), 64)
    with pytest.raises(ValueError, match="ld >= max_seq_len"):
        dsa.indexer_topk(_batch(), q, w, _keys(), 64, scores=torch.zeros((T, 200)))
    with pytest.raises(ValueError, match="indices must be"):
        dsa.indexer_topk(_batch(), q, w, _keys(), 64, scores=torch.zeros((T, 300)),
                         indices=torch.zeros((T, 32), dtype=torch.int32))
