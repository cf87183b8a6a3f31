"""MI355X sparse-attention decode: lightning indexer -> top-k -> sparse MLA.

Thin torch-facing binding of the C-ABI library ``libdsa.so`` (see
``include/dsa.h``). PyTorch only supplies device memory and the current
stream; every step runs in the library's HIP kernels. Each wrapper checks
dtypes, shapes, devices and contiguity (the batch's arrays against its
sequence count, and every per-row tensor, caller-supplied outputs included,
against the batch's ``total_q``, since the kernels size their work from it),
passes raw pointers, and raises :class:`DSAError` on a non-zero status.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

from ._lib import (  # noqa: F401
    DSA_BF16,
    DSA_F32,
    DSA_FP8_E4M3,
    DSAError,
    DsaBatch,
    DsaPagedCache,
    check,
    lib,
    status_str,
)

__all__ = [
    "Batch", "PagedCache", "DSAError", "indexer_scores", "topk", "sparse_mla_fwd",
    "topk_workspace_size", "sparse_mla_workspace_size", "abi_version", "kv_append",
    "page_scores", "page_topk", "page_topk_workspace_size", "indexer_page_scores",
    "sparse_mla_fwd_noalloc", "sparse_mla_fwd_qblocked", "sparse_mla_qblocked_workspace_size",
    "indexer_topk", "indexer_topk_state_size",
]

_DT = {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16, torch.uint8: DSA_FP8_E4M3,
       torch.float8_e4m3fn: DSA_FP8_E4M3}


def abi_version() -> int:
    return int(lib.dsa_abi_version())


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _rows(t: torch.Tensor, name: str, batch: "Batch", shape_tail=None) -> None:
    """The kernels size their work from batch.total_q: a per-row tensor must hold at
    least that many rows (and, when given, exactly the trailing shape)."""
    if t.dim() < 1 or t.shape[0] < batch.total_q:
        raise ValueError(f"{name} has {t.shape[0] if t.dim() else 0} rows, the batch has "
                         f"total_q = {batch.total_q}")
    if shape_tail is not None and tuple(t.shape[1:]) != tuple(shape_tail):
        raise ValueError(f"{name} must be [rows, {', '.join(map(str, shape_tail))}], got "
                         f"{tuple(t.shape)}")


@dataclass
class Batch:
    """Packed batch metadata: device arrays plus their host-side bounds."""

    block_table: torch.Tensor  # int32 [B, bt_stride]
    seq_lens: torch.Tensor  # int32 [B]
    cu_q: torch.Tensor  # int32 [B + 1]
    total_q: int
    max_seq_len: int
    max_q: int

    def c(self) -> DsaBatch:
        B = int(self.seq_lens.shape[0]) if self.seq_lens.dim() == 1 else -1
        if B < 0:
            raise ValueError("seq_lens must be [B]")
        if self.cu_q.dim() != 1 or self.cu_q.shape[0] != B + 1:
            raise ValueError(f"cu_q must be [B + 1] = [{B + 1}], got {tuple(self.cu_q.shape)}")
        if self.block_table.dim() != 2 or self.block_table.shape[0] != B:
            raise ValueError(f"block_table must be [B = {B}, bt_stride], got "
                             f"{tuple(self.block_table.shape)}")
        return DsaBatch(
            _dev(self.block_table, "block_table", torch.int32),
            _dev(self.seq_lens, "seq_lens", torch.int32),
            _dev(self.cu_q, "cu_q", torch.int32),
            int(self.seq_lens.shape[0]), int(self.block_table.shape[1]), int(self.total_q),
            int(self.max_seq_len), int(self.max_q))


@dataclass
class PagedCache:
    """A paged cache [num_pages, page_size, row] (+ fp32 scales [num_pages, page_size] for e4m3)."""

    data: torch.Tensor
    scale: Optional[torch.Tensor] = None

    def c(self) -> DsaPagedCache:
        if self.data.dim() != 3:
            raise ValueError("cache must be [num_pages, page_size, row_elems]")
        dt = _DT.get(self.data.dtype)
        if dt is None:
            raise TypeError(f"unsupported cache dtype {self.data.dtype}")
        sp = 0
        if dt == DSA_FP8_E4M3:
            if self.scale is None:
                raise ValueError("e4m3 cache needs per-token fp32 scales")
            if tuple(self.scale.shape) != tuple(self.data.shape[:2]):
                raise ValueError("scale must be [num_pages, page_size]")
            sp = _dev(self.scale, "scale", torch.float32)
        n, p, r = self.data.shape
        return DsaPagedCache(_dev(self.data, "cache"), sp, n, p, r, dt)


def indexer_scores(batch: Batch, q_idx: torch.Tensor, w: torch.Tensor, keys: PagedCache,
                   scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """I[r, s] = sum_j w[r, j] ReLU(q_idx[r, j] . k(s)) for s <= t_r; [T, ld] fp32 (rest untouched)."""
    T, H, D = q_idx.shape
    qd = _DT.get(q_idx.dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q_idx must be float32 or bfloat16")
    if tuple(w.shape) != (T, H):
        raise ValueError("w must be [T, n_heads]")
    _rows(q_idx, "q_idx", batch)
    if scores is None:
        scores = torch.empty((T, max(1, batch.max_seq_len)), dtype=torch.float32,
                             device=q_idx.device)
    if scores.dim() != 2 or scores.shape[0] != T:
        raise ValueError("scores must be [T, ld]")
    if scores.shape[1] < batch.max_seq_len:
        raise ValueError("scores rows must hold max_seq_len entries")
    b, kc = batch.c(), keys.c()
    check(lib.dsa_indexer_scores(ctypes.byref(b), _dev(q_idx, "q_idx"), qd,
                                 _dev(w, "w", torch.float32), H, D, ctypes.byref(kc),
                                 _dev(scores, "scores", torch.float32), scores.shape[1],
                                 _stream(q_idx.device)), "dsa_indexer_scores")
    return scores


def topk_workspace_size(total_q: int, max_seq_len: int, k: int) -> int:
    return int(lib.dsa_topk_workspace_size(total_q, max_seq_len, k))


def topk(batch: Batch, scores: torch.Tensor, k: int, indices: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[T, k] int32: the min(k, t_r + 1) best positions per row, ascending, then -1."""
    T = scores.shape[0]
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if tuple(indices.shape) != (T, k):
        raise ValueError("indices must be [T, k]")
    _rows(scores, "scores", batch)
    if scores.dim() != 2 or scores.shape[1] < batch.max_seq_len:
        raise ValueError("scores must be [T, ld] with ld >= max_seq_len")
    need = topk_workspace_size(batch.total_q, batch.max_seq_len, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    wp = 0 if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    b = batch.c()
    check(lib.dsa_topk(ctypes.byref(b), _dev(scores, "scores", torch.float32), scores.shape[1], k,
                       _dev(indices, "indices", torch.int32), wp, wb, _stream(scores.device)),
          "dsa_topk")
    return indices


def page_scores(batch: Batch, scores: torch.Tensor, page_size: int,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[T, ld_pages] fp32: max of each logical page's legal token scores (pages past t_r
    untouched)."""
    T = scores.shape[0]
    n_pages = max(1, -(-batch.max_seq_len // page_size))
    if out is None:
        out = torch.empty((T, n_pages), dtype=torch.float32, device=scores.device)
    if out.dim() != 2 or out.shape[0] != T or out.shape[1] < n_pages:
        raise ValueError("page scores must be [T, ld_pages] with ld_pages >= the page count")
    _rows(scores, "scores", batch)
    b = batch.c()
    check(lib.dsa_page_scores(ctypes.byref(b), _dev(scores, "scores", torch.float32),
                              scores.shape[1], page_size, _dev(out, "page_scores", torch.float32),
                              out.shape[1], _stream(scores.device)), "dsa_page_scores")
    return out


def indexer_page_scores(batch: Batch, q_idx: torch.Tensor, w: torch.Tensor, keys: PagedCache,
                        page_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[T, ld_pages] fp32 page maxima of the indexer scores, computed without writing token
    scores (the streamed-key configurations only; DSAError(UNSUPPORTED) otherwise)."""
    T, H, D = q_idx.shape
    qd = _DT.get(q_idx.dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q_idx must be float32 or bfloat16")
    if tuple(w.shape) != (T, H):
        raise ValueError("w must be [T, n_heads]")
    n_pages = max(1, -(-batch.max_seq_len // page_size))
    if out is None:
        out = torch.empty((T, n_pages), dtype=torch.float32, device=q_idx.device)
    if out.dim() != 2 or out.shape[0] != T or out.shape[1] < n_pages:
        raise ValueError("page scores must be [T, ld_pages] with ld_pages >= the page count")
    _rows(q_idx, "q_idx", batch)
    b, kc = batch.c(), keys.c()
    check(lib.dsa_indexer_page_scores(ctypes.byref(b), _dev(q_idx, "q_idx"), qd,
                                      _dev(w, "w", torch.float32), H, D, ctypes.byref(kc),
                                      page_size, _dev(out, "page_scores", torch.float32),
                                      out.shape[1], _stream(q_idx.device)),
          "dsa_indexer_page_scores")
    return out


def indexer_topk_state_size(total_q: int) -> int:
    return int(lib.dsa_indexer_topk_state_size(total_q))


def indexer_topk(batch: Batch, q_idx: torch.Tensor, w: torch.Tensor, keys: PagedCache, k: int,
                 scores: Optional[torch.Tensor] = None, indices: Optional[torch.Tensor] = None,
                 state: Optional[torch.Tensor] = None):
    """(scores [T, ld], indices [T, k]): indexer_scores then topk in one launch (decode rows
    of the streamed-key configurations; DSAError(UNSUPPORTED) otherwise). `state` must be
    zero-filled before its first call and is zero-filled again after each call; a new one is
    made when it is None."""
    T, H, D = q_idx.shape
    qd = _DT.get(q_idx.dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q_idx must be float32 or bfloat16")
    if tuple(w.shape) != (T, H):
        raise ValueError("w must be [T, n_heads]")
    _rows(q_idx, "q_idx", batch)
    dev = q_idx.device
    if scores is None:
        scores = torch.empty((T, max(1, batch.max_seq_len)), dtype=torch.float32, device=dev)
    if scores.dim() != 2 or scores.shape[0] != T or scores.shape[1] < batch.max_seq_len:
        raise ValueError("scores must be [T, ld] with ld >= max_seq_len")
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=dev)
    if tuple(indices.shape) != (T, k):
        raise ValueError("indices must be [T, k]")
    need = indexer_topk_state_size(batch.total_q)
    if state is None:
        state = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    b, kc = batch.c(), keys.c()
    check(lib.dsa_indexer_topk(ctypes.byref(b), _dev(q_idx, "q_idx"), qd,
                               _dev(w, "w", torch.float32), H, D, ctypes.byref(kc), k,
                               _dev(scores, "scores", torch.float32), scores.shape[1],
                               _dev(indices, "indices", torch.int32), _dev(state, "state"),
                               state.numel() * state.element_size(), _stream(dev)),
          "dsa_indexer_topk")
    return scores, indices


def page_topk_workspace_size(total_q: int, max_seq_len: int, page_size: int, kp: int) -> int:
    return int(lib.dsa_page_topk_workspace_size(total_q, max_seq_len, page_size, kp))


def page_topk(batch: Batch, page_scores: torch.Tensor, page_size: int, kp: int,
              pages: Optional[torch.Tensor] = None, indices: Optional[torch.Tensor] = None,
              want_indices: bool = True, workspace: Optional[torch.Tensor] = None):
    """(pages [T, kp], indices [T, kp * page_size] or None): the kp best pages per row
    (ascending, -1 padded) and their legal token positions."""
    T = page_scores.shape[0]
    dev = page_scores.device
    if pages is None:
        pages = torch.empty((T, kp), dtype=torch.int32, device=dev)
    if indices is None and want_indices:
        indices = torch.empty((T, kp * page_size), dtype=torch.int32, device=dev)
    if tuple(pages.shape) != (T, kp):
        raise ValueError("pages must be [T, kp]")
    if indices is not None and tuple(indices.shape) != (T, kp * page_size):
        raise ValueError("indices must be [T, kp * page_size]")
    _rows(page_scores, "page_scores", batch)
    need = page_topk_workspace_size(batch.total_q, batch.max_seq_len, page_size, kp)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wp = 0 if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    b = batch.c()
    check(lib.dsa_page_topk(ctypes.byref(b), _dev(page_scores, "page_scores", torch.float32),
                            page_scores.shape[1], page_size, kp, _dev(pages, "pages", torch.int32),
                            0 if indices is None else _dev(indices, "indices", torch.int32),
                            wp, wb, _stream(dev)), "dsa_page_topk")
    return pages, indices


def sparse_mla_workspace_size(total_q: int, n_heads: int, d_latent: int, k: int) -> int:
    return int(lib.dsa_sparse_mla_workspace_size(total_q, n_heads, d_latent, k))


def sparse_mla_fwd(batch: Batch, q: torch.Tensor, kv: PagedCache, indices: torch.Tensor,
                   d_latent: int, scale: float, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Absorbed sparse MLA: out [T, H, d_latent] fp32 and lse [T, H] fp32 (natural log)."""
    T, H, D = q.shape
    qd = _DT.get(q.dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q must be float32 or bfloat16")
    d_rope = D - d_latent
    if indices.dim() != 2:
        raise ValueError("indices must be [T, k]")
    k = indices.shape[1]
    _rows(q, "q", batch)
    _rows(indices, "indices", batch)
    if out is None:
        out = torch.empty((T, H, d_latent), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _rows(out, "out", batch, (H, d_latent))
    if lse is not None:
        _rows(lse, "lse", batch, (H,))
    need = sparse_mla_workspace_size(batch.total_q, H, d_latent, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp = 0 if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    b, kc = batch.c(), kv.c()
    check(lib.dsa_sparse_mla_fwd(ctypes.byref(b), _dev(q, "q"), qd, H, d_latent, d_rope,
                                 ctypes.byref(kc), _dev(indices, "indices", torch.int32), k,
                                 float(scale), _dev(out, "out", torch.float32),
                                 0 if lse is None else _dev(lse, "lse", torch.float32), wp, wb,
                                 _stream(q.device)), "dsa_sparse_mla_fwd")
    return out, lse


def sparse_mla_fwd_noalloc(batch: Batch, q: torch.Tensor, kv: PagedCache, indices: torch.Tensor,
                           d_latent: int, scale: float, out: torch.Tensor,
                           lse: Optional[torch.Tensor] = None):
    """sparse_mla_fwd with the split partials in the library's static per-GPU scratch
    array instead of a workspace (dsa_sparse_mla_fwd_noalloc): the caller passes the
    outputs, and neither the library nor this wrapper allocates. Calls that may overlap
    on one GPU race on the shared array."""
    T, H, D = q.shape
    qd = _DT.get(q.dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q must be float32 or bfloat16")
    if indices.dim() != 2:
        raise ValueError("indices must be [T, k]")
    k = indices.shape[1]
    _rows(q, "q", batch)
    _rows(indices, "indices", batch)
    _rows(out, "out", batch, (H, d_latent))
    if lse is not None:
        _rows(lse, "lse", batch, (H,))
    b, kc = batch.c(), kv.c()
    check(lib.dsa_sparse_mla_fwd_noalloc(ctypes.byref(b), _dev(q, "q"), qd, H, d_latent, D - d_latent,
                                         ctypes.byref(kc), _dev(indices, "indices", torch.int32), k,
                                         float(scale), _dev(out, "out", torch.float32),
                                         0 if lse is None else _dev(lse, "lse", torch.float32),
                                         _stream(q.device)), "dsa_sparse_mla_fwd_noalloc")
    return out, lse


def sparse_mla_qblocked_workspace_size(total_q: int, n_heads: int, k: int) -> int:
    return int(lib.dsa_sparse_mla_qblocked_workspace_size(total_q, n_heads, k))


def sparse_mla_fwd_qblocked(batch: Batch, q: torch.Tensor, kv: PagedCache, indices: torch.Tensor,
                            d_latent: int, scale: float, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, want_lse: bool = True):
    """Query-blocked sparse MLA (dsa_sparse_mla_fwd_qblocked): the same result as
    sparse_mla_fwd to rounding, each block of query rows loading the union of its
    selected rows once. Returns (out [T, H, d_latent], lse [T, H] or None)."""
    T, H, D = q.shape
    qd = _DT.get(q.dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q must be float32 or bfloat16")
    if indices.dim() != 2:
        raise ValueError("indices must be [T, k]")
    k = indices.shape[1]
    _rows(q, "q", batch)
    _rows(indices, "indices", batch)
    if out is None:
        out = torch.empty((T, H, d_latent), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _rows(out, "out", batch, (H, d_latent))
    if lse is not None:
        _rows(lse, "lse", batch, (H,))
    need = sparse_mla_qblocked_workspace_size(batch.total_q, H, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp = 0 if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    b, kc = batch.c(), kv.c()
    check(lib.dsa_sparse_mla_fwd_qblocked(ctypes.byref(b), _dev(q, "q"), qd, H, d_latent,
                                          D - d_latent, ctypes.byref(kc),
                                          _dev(indices, "indices", torch.int32), k, float(scale),
                                          _dev(out, "out", torch.float32),
                                          0 if lse is None else _dev(lse, "lse", torch.float32),
                                          wp, wb, _stream(q.device)), "dsa_sparse_mla_fwd_qblocked")
    return out, lse


def sparse_mla_layers_workspace_size(n_layers: int, total_q: int, n_heads: int, d_latent: int,
                                     k: int) -> int:
    return int(lib.dsa_sparse_mla_layers_workspace_size(n_layers, total_q, n_heads, d_latent, k))


def sparse_mla_fwd_layers(batch: Batch, qs: Sequence[torch.Tensor], kvs: Sequence[PagedCache],
                          indices: torch.Tensor, d_latent: int, scale: float,
                          outs: Optional[Sequence[torch.Tensor]] = None,
                          lses: Optional[Sequence[torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None,
                          want_lse: bool = True):
    """IndexShare: sparse_mla_fwd for several layers on one index list, as one call.
    Returns (outs, lses), lists of per-layer [T, H, d_latent] and [T, H] fp32 tensors;
    an entry of `lses` may be None (no lse for that layer)."""
    n = len(qs)
    if n != len(kvs) or n < 1:
        raise ValueError("one cache per query tensor, at least one layer")
    if (outs is not None and len(outs) != n) or (lses is not None and len(lses) != n):
        raise ValueError("outs and lses need one entry per layer")
    T, H, D = qs[0].shape
    qd = _DT.get(qs[0].dtype)
    if qd not in (DSA_F32, DSA_BF16):
        raise TypeError("q must be float32 or bfloat16")
    if any(tuple(q.shape) != (T, H, D) or q.dtype != qs[0].dtype for q in qs):
        raise ValueError("every layer's q must have the same shape and dtype")
    d_rope = D - d_latent
    if indices.dim() != 2:
        raise ValueError("indices must be [T, k]")
    k = indices.shape[1]
    dev = qs[0].device
    _rows(qs[0], "q", batch)
    _rows(indices, "indices", batch)
    if outs is None:
        outs = [torch.empty((T, H, d_latent), dtype=torch.float32, device=dev) for _ in range(n)]
    if lses is None and want_lse:
        lses = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(n)]
    for o in outs:
        _rows(o, "out", batch, (H, d_latent))
    for x in lses or []:
        if x is not None:
            _rows(x, "lse", batch, (H,))
    need = sparse_mla_layers_workspace_size(n, batch.total_q, H, d_latent, k)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wp = 0 if workspace is None else _dev(workspace, "workspace")
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    q_arr = (ctypes.c_void_p * n)(*[_dev(q, "q") for q in qs])
    o_arr = (ctypes.c_void_p * n)(*[_dev(o, "out", torch.float32) for o in outs])
    l_arr = None if lses is None else (ctypes.c_void_p * n)(
        *[None if x is None else _dev(x, "lse", torch.float32) for x in lses])
    kv_arr = (DsaPagedCache * n)(*[kv.c() for kv in kvs])
    b = batch.c()
    check(lib.dsa_sparse_mla_fwd_layers(
        ctypes.byref(b), n, ctypes.cast(q_arr, ctypes.c_void_p), qd, H, d_latent, d_rope,
        kv_arr, _dev(indices, "indices", torch.int32), k, float(scale),
        ctypes.cast(o_arr, ctypes.c_void_p),
        None if l_arr is None else ctypes.cast(l_arr, ctypes.c_void_p), wp, wb, _stream(dev)),
        "dsa_sparse_mla_fwd_layers")
    return list(outs), (None if lses is None else list(lses))


def kv_append(slot_mapping: torch.Tensor, latent: Optional[torch.Tensor] = None,
              kv: Optional[PagedCache] = None, idx_keys: Optional[torch.Tensor] = None,
              k_idx: Optional[PagedCache] = None) -> None:
    """Write new tokens into paged caches in place: token i to slot slot_mapping[i]
    (page * page_size + offset; negative or out-of-pool slots are skipped). Latent
    rows are copied; indexer keys are copied, or quantised per token for an e4m3
    cache (scale = max|k| / 448)."""
    n = int(slot_mapping.numel())
    if (latent is None) != (kv is None) or (idx_keys is None) != (k_idx is None):
        raise ValueError("each cache needs its new rows and each set of rows its cache")
    sp = _dev(slot_mapping, "slot_mapping", torch.int32)
    lp, kp, kd = 0, 0, DSA_BF16
    kvc = ctypes.POINTER(DsaPagedCache)()
    kic = ctypes.POINTER(DsaPagedCache)()
    if kv is not None:
        if latent.dim() != 2 or latent.shape[0] != n or latent.shape[1] != kv.data.shape[2]:
            raise ValueError("latent must be [n_tokens, row_elems]")
        if latent.dtype != kv.data.dtype:
            raise TypeError("latent rows must have the latent cache's dtype")
        lp = _dev(latent, "latent")
        kvs = kv.c()
        kvc = ctypes.pointer(kvs)
    if k_idx is not None:
        if idx_keys.dim() != 2 or idx_keys.shape[0] != n or idx_keys.shape[1] != k_idx.data.shape[2]:
            raise ValueError("idx_keys must be [n_tokens, row_elems]")
        kd = _DT.get(idx_keys.dtype)
        if kd not in (DSA_F32, DSA_BF16):
            raise TypeError("idx_keys must be float32 or bfloat16")
        kp = _dev(idx_keys, "idx_keys")
        kis = k_idx.c()
        kic = ctypes.pointer(kis)
    dev = slot_mapping.device
    check(lib.dsa_kv_append(sp, n, lp, kvc, kp, kd, kic, _stream(dev)), "dsa_kv_append")
