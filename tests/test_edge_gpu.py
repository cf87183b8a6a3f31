"""GPU edge cases of the binding: an empty batch (every sequence with zero
query rows) passes through every call of both selection routes and returns
empty outputs; the library enqueues nothing for it."""

import pytest
import torch

import sparse_attention_decode_lightning_amd as dsa

pytestmark = pytest.mark.gpu


def test_empty_batch_through_every_call():
    dev = torch.device("cuda:0")
    print("[edge] empty batch", flush=True)
    i32 = dict(dtype=torch.int32, device=dev)
    batch = dsa.Batch(torch.zeros((2, 4), **i32), torch.tensor([70, 5], **i32),
                      torch.zeros(3, **i32), 0, 70, 0)
    keys = dsa.PagedCache(torch.zeros((8, 64, 128), dtype=torch.bfloat16, device=dev))
    kv = dsa.PagedCache(torch.zeros((8, 64, 576), dtype=torch.bfloat16, device=dev))
    q_idx = torch.empty((0, 32, 128), dtype=torch.bfloat16, device=dev)
    w = torch.empty((0, 32), dtype=torch.float32, device=dev)
    scores = dsa.indexer_scores(batch, q_idx, w, keys)
    idx = dsa.topk(batch, scores, 64)
    out, lse = dsa.sparse_mla_fwd(batch, torch.empty((0, 64, 576), dtype=torch.bfloat16, device=dev),
                                  kv, idx, 512, 0.0625)
    pscores = dsa.page_scores(batch, scores, 64)
    fused = dsa.indexer_page_scores(batch, q_idx, w, keys, 64)
    pages, pidx = dsa.page_topk(batch, pscores, 64, 2)
    torch.cuda.synchronize()
    assert scores.shape[0] == idx.shape[0] == out.shape[0] == lse.shape[0] == 0
    assert pscores.shape[0] == fused.shape[0] == pages.shape[0] == pidx.shape[0] == 0
    assert tuple(out.shape) == (0, 64, 512) and tuple(pidx.shape) == (0, 128)
