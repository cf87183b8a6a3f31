"""Seeded synthetic workloads in the paged layout of the decode path.

Each workload mirrors one shape the GLM-5.2 pages describe (64 MLA heads over
a 512-d latent plus a 64-d RoPE key per cached token, a 32-head x 128-d
lightning indexer with one shared key per token, top-2048 selection), filled
with N(0,1) data because no trained weights or real caches are available.

Layout (shared by the HIP library and the CPU oracle):

* ``block_table[b, j]``: physical page of logical page ``j`` of sequence ``b``.
  Pages are a random permutation of a pool that also holds unused pages.
* ``seq_lens[b]``: KV length of sequence ``b`` *including* this step's queries.
* ``cu_q[b]``: first query row of sequence ``b``; row ``cu_q[b] + i`` sits at
  absolute position ``seq_lens[b] - q_b + i``.
* indexer keys ``k_cache[page, slot, D_I]`` (f32, bf16, or OCP e4m3fn bytes
  with a per-token fp32 scale ``k_scale[page, slot]``);
* latent rows ``kv_cache[page, slot, D_L + D_R]`` (latent first, RoPE key last).

Unused pages, the slots past each sequence's length in its last page, and the
block-table entries past a sequence's last page are poisoned (NaN, or the
e4m3fn NaN byte 0x7F) so any read outside the valid region shows up as NaN.

Nothing here computes scores, selections or attention.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence, Union

import torch

E4M3_MAX = 448.0
E4M3_NAN_BYTE = 0x7F

LenSpec = Union[int, Sequence[int], tuple]


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic batch."""

    name: str
    seed: int
    batch: int
    lens: LenSpec  # int, explicit tuple, or ("uniform", lo, hi) inclusive
    q_per_seq: Union[int, Sequence[int]]
    page_size: int
    idx_heads: int
    idx_dim: int
    idx_q_dtype: str  # "f32" | "bf16"
    idx_k_dtype: str  # "f32" | "bf16" | "fp8"
    w_std: float
    topk: int
    mla_heads: int
    d_latent: int
    d_rope: int
    mla_dtype: str  # "f32" | "bf16"
    scale: float
    n_layers: int = 1
    spare_frac: float = 0.125
    description: str = ""

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed=1, batch=1, lens=256, q_per_seq=1, page_size=16,
        idx_heads=4, idx_dim=32, idx_q_dtype="f32", idx_k_dtype="f32",
        w_std=1.0 / math.sqrt(4), topk=64, mla_heads=8, d_latent=64, d_rope=16,
        mla_dtype="f32", scale=float(1.0 / math.sqrt(48)), n_layers=1, spare_frac=0.25,
        description="tiny decode: B=1, L=256, f32 indexer 4x32, top-64, 8-head 64+16 f32 MLA, page 16",
    ),
    "decode_b32_l8k": Workload(
        name="decode_b32_l8k", seed=2, batch=32, lens=8192, q_per_seq=1, page_size=64,
        idx_heads=32, idx_dim=128, idx_q_dtype="bf16", idx_k_dtype="bf16",
        w_std=1.0 / math.sqrt(32), topk=2048, mla_heads=64, d_latent=512, d_rope=64,
        mla_dtype="bf16", scale=1.0 / 16.0, n_layers=1,
        description="decode B=32, L=8192, bf16 indexer 32x128, top-2048, 64-head 512+64 bf16 MLA, page 64",
    ),
    "indexshare_b64": Workload(
        name="indexshare_b64", seed=3, batch=64, lens=("uniform", 2048, 131072), q_per_seq=1,
        page_size=64, idx_heads=32, idx_dim=128, idx_q_dtype="bf16", idx_k_dtype="fp8",
        w_std=1.0 / math.sqrt(32), topk=2048, mla_heads=64, d_latent=512, d_rope=64,
        mla_dtype="bf16", scale=1.0 / 16.0, n_layers=3,
        description="decode B=64, L~U[2048,131072], fp8 indexer keys, top-2048 shared by 3 MLA layers",
    ),
    "prefill_q4k_l32k": Workload(
        name="prefill_q4k_l32k", seed=4, batch=1, lens=32768, q_per_seq=4096, page_size=128,
        idx_heads=32, idx_dim=128, idx_q_dtype="bf16", idx_k_dtype="bf16",
        w_std=1.0 / math.sqrt(32), topk=2048, mla_heads=64, d_latent=512, d_rope=64,
        mla_dtype="bf16", scale=1.0 / 16.0, n_layers=1,
        description="prefill chunk: 4096 queries after 28672 cached tokens, bf16 indexer, page 128",
    ),
    "verify_b8_l240k": Workload(
        name="verify_b8_l240k", seed=5, batch=8, lens=245760, q_per_seq=4, page_size=64,
        idx_heads=32, idx_dim=128, idx_q_dtype="bf16", idx_k_dtype="fp8",
        w_std=1.0 / math.sqrt(32), topk=2048, mla_heads=64, d_latent=512, d_rope=64,
        mla_dtype="bf16", scale=1.0 / 16.0, n_layers=1,
        description="long-context draft verify: B=8, L=245760, 4 causal queries/seq, fp8 keys, page 64",
    ),
}


def small_variant(base: str | Workload, **kw) -> Workload:
    """A copy of a workload with some fields overridden (used for small parity cases)."""
    wl = WORKLOADS[base] if isinstance(base, str) else base
    return wl.replace(**kw)


@dataclass
class Inputs:
    """Device-or-host tensors of one workload; see the module docstring for layouts."""

    wl: Workload
    seq_lens: torch.Tensor  # int32 [B]
    q_lens: torch.Tensor  # int32 [B]
    cu_q: torch.Tensor  # int32 [B+1]
    block_table: torch.Tensor  # int32 [B, bt_stride]
    q_idx: torch.Tensor  # [T, H_I, D_I] f32|bf16
    w: torch.Tensor  # [T, H_I] f32
    k_cache: torch.Tensor  # [pool, P, D_I] f32|bf16|uint8
    k_scale: Optional[torch.Tensor]  # [pool, P] f32 (fp8 keys only)
    q_mla: list = field(default_factory=list)  # per layer [T, H, D_L+D_R]
    kv_cache: list = field(default_factory=list)  # per layer [pool, P, D_L+D_R]
    max_seq_len: int = 0
    max_q: int = 0
    total_q: int = 0
    num_pages: int = 0
    seq_lens_host: list = field(default_factory=list)
    q_lens_host: list = field(default_factory=list)

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])


_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _draw_lens(wl: Workload, g: torch.Generator) -> list:
    spec = wl.lens
    if isinstance(spec, int):
        return [spec] * wl.batch
    if isinstance(spec, tuple) and len(spec) == 3 and spec[0] == "uniform":
        lo, hi = int(spec[1]), int(spec[2])
        return torch.randint(lo, hi + 1, (wl.batch,), generator=g).tolist()
    lens = [int(x) for x in spec]
    assert len(lens) == wl.batch
    return lens


def _q_lens(wl: Workload) -> list:
    if isinstance(wl.q_per_seq, int):
        return [wl.q_per_seq] * wl.batch
    q = [int(x) for x in wl.q_per_seq]
    assert len(q) == wl.batch
    return q


def _randn(shape, g, device, dtype, chunk_rows=2048):
    """N(0,1) in ``dtype``, drawn in fp32 in chunks along dim 0 to bound temporaries."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n = shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device,
                               dtype=torch.float32).to(dtype)
    return out


def _fp8_keys(shape, g, device, chunk_rows=2048):
    """Per-token e4m3fn bytes and fp32 scales: sigma = amax|k| / 448, byte = e4m3fn(k / sigma)."""
    pool, P, D = shape
    data = torch.empty((pool, P, D), dtype=torch.uint8, device=device)
    scale = torch.empty((pool, P), dtype=torch.float32, device=device)
    for s in range(0, pool, chunk_rows):
        e = min(pool, s + chunk_rows)
        k = torch.randn((e - s, P, D), generator=g, device=device, dtype=torch.float32)
        sig = k.abs().amax(dim=-1) / E4M3_MAX
        sig = torch.where(sig > 0, sig, torch.ones_like(sig))
        q = (k / sig[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
        data[s:e] = q.to(torch.float8_e4m3fn).view(torch.uint8)
        scale[s:e] = sig
    return data, scale


def make_inputs(wl: Workload, device: str = "cpu", poison: bool = True) -> Inputs:
    """Draw one batch of ``wl`` with a CPU generator seeded by ``wl.seed``.

    Metadata (lengths, block table) is always drawn on the CPU. Bulk data is
    drawn on ``device`` with a generator of that device seeded the same way, so
    a CPU draw is reproducible anywhere and a GPU draw is reproducible on the
    same GPU software stack.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed)
    gd = g if device == "cpu" else torch.Generator(device=device)
    if device != "cpu":
        gd.manual_seed(wl.seed + 1000003)

    lens = _draw_lens(wl, g)
    qlens = _q_lens(wl)
    for L, q in zip(lens, qlens):
        assert L >= q >= 0, (L, q)
    P = wl.page_size
    pages_per_seq = [(L + P - 1) // P for L in lens]
    used = sum(pages_per_seq)
    pool = used + int(math.ceil(used * wl.spare_frac))
    bt_stride = max(1, max(pages_per_seq))
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    spare_pages = perm[used:]
    poison_page = int(spare_pages[0]) if len(spare_pages) > 0 else 0
    bt = torch.full((wl.batch, bt_stride), poison_page, dtype=torch.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        bt[b, :n] = perm[off:off + n]
        off += n
    cu = [0]
    for q in qlens:
        cu.append(cu[-1] + q)
    T = cu[-1]

    # indexer inputs (drawn on the CPU generator for the small tensors)
    q_idx = torch.randn((T, wl.idx_heads, wl.idx_dim), generator=g, dtype=torch.float32)
    q_idx = q_idx.to(_TORCH_DT[wl.idx_q_dtype])
    w = torch.randn((T, wl.idx_heads), generator=g, dtype=torch.float32) * wl.w_std
    q_mla = []
    for _ in range(wl.n_layers):
        q = torch.randn((T, wl.mla_heads, wl.d_latent + wl.d_rope), generator=g,
                        dtype=torch.float32)
        q_mla.append(q.to(_TORCH_DT[wl.mla_dtype]).to(device))

    # bulk caches
    if wl.idx_k_dtype == "fp8":
        k_cache, k_scale = _fp8_keys((pool, P, wl.idx_dim), gd, device)
    else:
        k_cache = _randn((pool, P, wl.idx_dim), gd, device, _TORCH_DT[wl.idx_k_dtype])
        k_scale = None
    kv = [_randn((pool, P, wl.d_latent + wl.d_rope), gd, device, _TORCH_DT[wl.mla_dtype])
          for _ in range(wl.n_layers)]

    if poison and pool > 0:
        bad = torch.zeros(pool, P, dtype=torch.bool)
        if len(spare_pages) > 0:
            bad[spare_pages.long()] = True
        for b, L in enumerate(lens):
            n = pages_per_seq[b]
            if n > 0 and L % P:
                bad[int(bt[b, n - 1]), L % P:] = True
        bad = bad.to(device)
        if wl.idx_k_dtype == "fp8":
            k_cache[bad] = E4M3_NAN_BYTE
            k_scale[bad] = float("nan")
        else:
            k_cache[bad] = float("nan")
        for c in kv:
            c[bad] = float("nan")

    return Inputs(
        wl=wl,
        seq_lens=torch.tensor(lens, dtype=torch.int32).to(device),
        q_lens=torch.tensor(qlens, dtype=torch.int32).to(device),
        cu_q=torch.tensor(cu, dtype=torch.int32).to(device),
        block_table=bt.to(device),
        q_idx=q_idx.to(device),
        w=w.to(device),
        k_cache=k_cache,
        k_scale=k_scale,
        q_mla=q_mla,
        kv_cache=kv,
        max_seq_len=max(lens) if lens else 0,
        max_q=max(qlens) if qlens else 0,
        total_q=T,
        num_pages=pool,
        seq_lens_host=list(lens),
        q_lens_host=list(qlens),
    )


# --------------------------------------------------------------------------
# host views: raw stored elements as numpy arrays (bit views, no arithmetic)
# --------------------------------------------------------------------------


def raw_numpy(t: torch.Tensor, tag: str):
    """Stored elements of ``t`` as numpy: uint16 bit patterns for bf16, else as stored."""
    import numpy as np

    t = t.detach().contiguous().cpu()
    if tag == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    if tag == "fp8":
        return t.numpy().astype(np.uint8, copy=False)
    return t.numpy()


class PagedRows:
    """Numpy-style ``cache[pages, slots]`` reads of a (possibly device) cache tensor.

    Lets a host-side reader fetch only the rows it needs from a cache that is
    too large to copy whole; the gather is plain tensor indexing.
    """

    def __init__(self, t: torch.Tensor, tag: str):
        self.t = t
        self.tag = tag
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        pages, slots = key
        p = torch.as_tensor(pages, dtype=torch.long).to(self.t.device)
        s = torch.as_tensor(slots, dtype=torch.long).to(self.t.device)
        return raw_numpy(self.t[p, s], self.tag)


def host_view(inp: Inputs, lazy: bool = False) -> dict:
    """Everything a host-side reader needs, as numpy arrays of raw stored elements.

    With ``lazy`` the big caches stay where they are and are read row by row
    through :class:`PagedRows`.
    """
    wl = inp.wl
    kdt = wl.idx_k_dtype

    def cache(t, tag):
        return PagedRows(t, tag) if lazy else raw_numpy(t, tag)

    return {
        "seq_lens": list(inp.seq_lens_host),
        "q_lens": list(inp.q_lens_host),
        "block_table": raw_numpy(inp.block_table, "i32"),
        "page_size": wl.page_size,
        "q_idx": raw_numpy(inp.q_idx, wl.idx_q_dtype),
        "idx_q_dtype": wl.idx_q_dtype,
        "w": raw_numpy(inp.w, "f32"),
        "k_cache": cache(inp.k_cache, kdt),
        "k_scale": None if inp.k_scale is None else cache(inp.k_scale, "f32"),
        "idx_k_dtype": kdt,
        "q_mla": [raw_numpy(q, wl.mla_dtype) for q in inp.q_mla],
        "kv_cache": [cache(c, wl.mla_dtype) for c in inp.kv_cache],
        "mla_dtype": wl.mla_dtype,
        "d_latent": wl.d_latent,
        "scale": wl.scale,
        "topk": wl.topk,
    }


def to_device(inp: Inputs, device) -> Inputs:
    """A copy of ``inp`` with every tensor moved to ``device`` (host metadata kept)."""
    mv = lambda t: None if t is None else t.to(device)  # noqa: E731
    return dataclasses.replace(
        inp, seq_lens=mv(inp.seq_lens), q_lens=mv(inp.q_lens), cu_q=mv(inp.cu_q),
        block_table=mv(inp.block_table), q_idx=mv(inp.q_idx), w=mv(inp.w),
        k_cache=mv(inp.k_cache), k_scale=mv(inp.k_scale),
        q_mla=[mv(q) for q in inp.q_mla], kv_cache=[mv(c) for c in inp.kv_cache])


# --------------------------------------------------------------------------
# selection shapes for attention-only runs (indices drawn, not computed)
# --------------------------------------------------------------------------


def locality_indices(seq_lens, q_lens, k: int, page_size: int, block: int, hot_pages: int,
                     seed: int) -> torch.Tensor:
    """Locality-shaped selections: int32 [T, k] index lists in the layout the top-k
    writes (valid positions ascending, then -1).

    The query rows of each sequence are taken in blocks of ``block`` consecutive
    rows; a block draws ``hot_pages`` distinct logical pages among those its first
    row can see, and each of its rows draws min(k, n) distinct positions among the
    n positions of those pages it can see (position <= its own). Neighbouring
    queries thus select overlapping rows, the shape in which loading a block's
    union once pays. Uniform-random selections are the other shape (the top-k of
    random scores)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    T = sum(q_lens)
    out = torch.full((T, k), -1, dtype=torch.int32)
    r = 0
    for L, q in zip(seq_lens, q_lens):
        for i0 in range(0, q, block):
            t0 = L - q + i0
            n_pages = t0 // page_size + 1
            pages = torch.randperm(n_pages, generator=g)[: min(hot_pages, n_pages)]
            cand = (pages[:, None] * page_size + torch.arange(page_size)[None, :]).reshape(-1)
            for i in range(i0, min(q, i0 + block)):
                t = L - q + i
                legal = cand[cand <= t]
                pick = legal[torch.randperm(legal.numel(), generator=g)[: min(k, legal.numel())]]
                sel = torch.sort(pick).values.to(torch.int32)
                out[r + i, : sel.numel()] = sel
        r += q
    return out
