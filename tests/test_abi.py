"""The C-ABI library: it loads, exports what include/dsa.h declares, lays out its
structs as C does, and rejects bad arguments with status codes before touching
the GPU (CPU only; no kernel is launched here)."""

import ctypes
import os
import subprocess
import tempfile

import pytest

from sparse_attention_decode_lightning_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # an aligned address that validation rejects before any use


def test_every_declared_symbol_is_exported():
    names = L.declared_functions()
    assert set(names) >= {"dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_fwd",
                          "dsa_topk_workspace_size", "dsa_sparse_mla_workspace_size",
                          "dsa_status_str", "dsa_abi_version"}
    for n in names:
        assert hasattr(L.lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_bench_probe_library_exports_its_header():
    """include/dsa_bench.h (the benchmark's read-stream probe) is exported by
    libdsa_bench.so, and it rejects bad arguments before any launch."""
    import re
    text = open(os.path.join(ROOT, "include", "dsa_bench.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))
    assert names == ["dsa_bench_read", "dsa_bench_read_blocks"]
    path = os.path.join(os.path.dirname(L.LIB_PATH), "libdsa_bench.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported
    lib = ctypes.CDLL(path)
    lib.dsa_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    assert lib.dsa_bench_read(None, 16, FAKE, None) == 1
    assert lib.dsa_bench_read(FAKE, 0, FAKE, None) == 1
    assert lib.dsa_bench_read(FAKE + 4, 16, FAKE, None) == 2


def test_abi_version_and_status_strings():
    assert L.lib.dsa_abi_version() == 1
    for code, name in L.STATUS_NAMES.items():
        assert L.status_str(code).startswith(name)


def test_struct_layout_matches_c():
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "dsa.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(dsa_batch), offsetof(dsa_batch, batch),
         offsetof(dsa_batch, max_q), sizeof(dsa_paged_cache),
         offsetof(dsa_paged_cache, num_pages), offsetof(dsa_paged_cache, dtype));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "l")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe],
                       check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    assert got == [ctypes.sizeof(L.DsaBatch), L.DsaBatch.batch.offset, L.DsaBatch.max_q.offset,
                   ctypes.sizeof(L.DsaPagedCache), L.DsaPagedCache.num_pages.offset,
                   L.DsaPagedCache.dtype.offset]


def _batch(**kw):
    d = dict(block_table=FAKE, seq_lens=FAKE, cu_q=FAKE, batch=2, bt_stride=4, total_q=2,
             max_seq_len=200, max_q=1)
    d.update(kw)
    return L.DsaBatch(**d)


def _cache(**kw):
    d = dict(data=FAKE, scale=FAKE, num_pages=10, page_size=64, row_elems=128, dtype=L.DSA_BF16)
    d.update(kw)
    return L.DsaPagedCache(**d)


def _idx(b=None, q=FAKE, qd=L.DSA_BF16, w=FAKE, H=32, D=128, c=None, s=FAKE, ld=256):
    b = _batch() if b is None else b
    c = _cache() if c is None else c
    return L.lib.dsa_indexer_scores(ctypes.byref(b) if b is not False else None, q, qd, w, H, D,
                                    ctypes.byref(c) if c is not False else None, s, ld, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=False), 1), (dict(q=None), 1), (dict(w=None), 1), (dict(s=None), 1),
    (dict(c=False), 1), (dict(c=_cache(data=None)), 1),
    (dict(c=_cache(dtype=L.DSA_FP8_E4M3, row_elems=128, scale=None)), 1),
    (dict(b=_batch(seq_lens=None)), 1),
    (dict(ld=199), 2), (dict(H=0), 2), (dict(D=64), 2), (dict(c=_cache(page_size=0)), 2),
    (dict(c=_cache(num_pages=0)), 2), (dict(b=_batch(bt_stride=3)), 2),
    (dict(b=_batch(max_q=3)), 2), (dict(b=_batch(batch=-1)), 2), (dict(q=FAKE + 8), 2),
    (dict(qd=7), 3), (dict(c=_cache(dtype=9)), 3), (dict(qd=L.DSA_F32), 3),
    (dict(c=_cache(dtype=L.DSA_F32)), 3),
])
def test_indexer_rejects_bad_arguments(kw, code):
    assert _idx(**kw) == code


def _itk(b=None, q=FAKE, qd=L.DSA_BF16, w=FAKE, H=32, D=128, c=None, k=64, s=FAKE, ld=256,
         idx=FAKE, st=FAKE, stb=1 << 30):
    b = _batch() if b is None else b
    c = _cache() if c is None else c
    return L.lib.dsa_indexer_topk(ctypes.byref(b) if b is not False else None, q, qd, w, H, D,
                                  ctypes.byref(c) if c is not False else None, k, s, ld, idx,
                                  st, stb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=False), 1), (dict(q=None), 1), (dict(w=None), 1), (dict(s=None), 1),
    (dict(idx=None), 1), (dict(c=False), 1),
    (dict(k=0), 2), (dict(ld=199), 2), (dict(H=0), 2), (dict(D=64), 2), (dict(idx=FAKE + 2), 2),
    (dict(qd=7), 3), (dict(c=_cache(dtype=9)), 3),
    # valid, but outside the fused shapes
    (dict(H=24), 5), (dict(c=_cache(page_size=48), b=_batch(bt_stride=5)), 5),
    (dict(b=_batch(max_q=2)), 5),
    (dict(b=_batch(max_seq_len=16385, bt_stride=300), ld=16385), 5),
    (dict(qd=L.DSA_F32, c=_cache(dtype=L.DSA_F32)), 5),
    # the per-row state
    (dict(st=None), 4), (dict(stb=2 * 2112 * 4 - 1), 4), (dict(st=FAKE + 16), 4),
])
def test_indexer_topk_rejects_bad_arguments(kw, code):
    assert _itk(**kw) == code


def test_indexer_topk_state_size():
    assert L.lib.dsa_indexer_topk_state_size(0) == 0
    assert L.lib.dsa_indexer_topk_state_size(3) == 3 * (64 + 2048) * 4
    b = L.DsaBatch(block_table=None, seq_lens=None, cu_q=None, batch=0, bt_stride=0, total_q=0,
                   max_seq_len=0, max_q=0)
    assert _itk(b=b, q=None, w=None, s=None, idx=None, st=None, stb=0, ld=1) == 0


def _topk(b=None, s=FAKE, ld=256, k=64, idx=FAKE, ws=None, wsb=0):
    b = _batch() if b is None else b
    return L.lib.dsa_topk(ctypes.byref(b) if b is not False else None, s, ld, k, idx, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=False), 1), (dict(s=None), 1), (dict(idx=None), 1),
    (dict(k=0), 2), (dict(ld=100), 2), (dict(idx=FAKE + 2), 2), (dict(b=_batch(total_q=-1)), 2),
    (dict(b=_batch(max_seq_len=100000, bt_stride=2000), ld=100000, k=2048), 4),
    (dict(b=_batch(max_seq_len=100000, bt_stride=2000), ld=100000, k=2048, ws=FAKE, wsb=16), 4),
    (dict(b=_batch(max_seq_len=1 << 21, bt_stride=1 << 16), ld=1 << 21, k=2048), 5),
])
def test_topk_rejects_bad_arguments(kw, code):
    assert _topk(**kw) == code


def _mla(b=None, q=FAKE, qd=L.DSA_BF16, H=64, DL=512, DR=64, c=None, idx=FAKE, k=2048,
         scale=0.0625, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40):
    b = _batch() if b is None else b
    c = _cache(row_elems=576) if c is None else c
    return L.lib.dsa_sparse_mla_fwd(ctypes.byref(b) if b is not False else None, q, qd, H, DL, DR,
                                    ctypes.byref(c) if c is not False else None, idx, k, scale,
                                    out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=False), 1), (dict(q=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(c=False), 1),
    (dict(DR=32), 2), (dict(k=0), 2), (dict(scale=float("nan")), 2), (dict(H=0), 2),
    (dict(scale=0.0), 2), (dict(scale=-0.0625), 2), (dict(scale=float("inf")), 2),
    (dict(out=FAKE + 4), 2),
    (dict(qd=L.DSA_F32), 3), (dict(c=_cache(row_elems=576, dtype=L.DSA_FP8_E4M3)), 3),
    (dict(ws=None), 4), (dict(wsb=16), 4),
    (dict(qd=L.DSA_F32, c=_cache(row_elems=2048 + 64, dtype=L.DSA_F32), DL=2048), 5),
])
def test_mla_rejects_bad_arguments(kw, code):
    assert _mla(**kw) == code


def _mla_noalloc(b=None, q=FAKE, qd=L.DSA_BF16, H=64, DL=512, DR=64, c=None, idx=FAKE, k=2048,
                 scale=0.0625, out=FAKE, lse=FAKE):
    b = _batch() if b is None else b
    c = _cache(row_elems=576) if c is None else c
    return L.lib.dsa_sparse_mla_fwd_noalloc(ctypes.byref(b) if b is not False else None, q, qd, H,
                                            DL, DR, ctypes.byref(c) if c is not False else None,
                                            idx, k, scale, out, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=False), 1), (dict(q=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(c=False), 1), (dict(DR=32), 2), (dict(k=0), 2), (dict(scale=0.0), 2),
    (dict(out=FAKE + 4), 2), (dict(qd=L.DSA_F32), 3),
    # partials beyond the static scratch array: 32 rows x 32 splits x 64 x 514 fp32
    (dict(b=_batch(batch=32, total_q=32, max_q=1, max_seq_len=70000, bt_stride=1100),
          k=65536), 4),
])
def test_mla_noalloc_rejects_bad_arguments(kw, code):
    """The allocation-free variant validates like dsa_sparse_mla_fwd and rejects a call
    whose partials would not fit the library's scratch array, before any HIP call."""
    assert _mla_noalloc(**kw) == code


def test_mla_noalloc_limit_covers_every_decode_batch_at_k2048():
    assert max(L.lib.dsa_sparse_mla_workspace_size(t, 64, 512, 2048) for t in range(1, 1025)) \
        <= L.DSA_MLA_NOALLOC_SCRATCH_BYTES
    assert L.lib.dsa_sparse_mla_workspace_size(32, 64, 512, 65536) > L.DSA_MLA_NOALLOC_SCRATCH_BYTES


def _mla_qb(b=None, q=FAKE, qd=L.DSA_BF16, H=64, DL=512, DR=64, c=None, idx=FAKE, k=2048,
            scale=0.0625, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40):
    b = _batch() if b is None else b
    c = _cache(row_elems=576) if c is None else c
    return L.lib.dsa_sparse_mla_fwd_qblocked(ctypes.byref(b) if b is not False else None, q, qd, H,
                                             DL, DR, ctypes.byref(c) if c is not False else None,
                                             idx, k, scale, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=False), 1), (dict(q=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(c=False), 1), (dict(k=0), 2), (dict(scale=0.0), 2), (dict(scale=float("nan")), 2),
    (dict(out=FAKE + 4), 2), (dict(DR=32), 2), (dict(qd=L.DSA_F32), 3),
    (dict(ws=None), 4), (dict(wsb=16), 4), (dict(ws=FAKE + 8), 4),
    # head counts other than 8 or a multiple of 16 up to 64, other row widths,
    # or unions over 2^20 slots (QB k) are not supported
    (dict(H=12), 5), (dict(H=128), 5), (dict(H=4), 5), (dict(k=(1 << 18) + 1), 5),
    (dict(H=8, k=(1 << 17) + 1), 5),
    (dict(qd=L.DSA_F32, c=_cache(row_elems=576, dtype=L.DSA_F32)), 5),
    (dict(b=_batch(max_seq_len=1 << 29, bt_stride=(1 << 29) // 64)), 5),
])
def test_mla_qblocked_rejects_bad_arguments(kw, code):
    assert _mla_qb(**kw) == code


def test_mla_qblocked_workspace_is_one_union_per_block():
    # 4-query blocks (16..64 heads) or 8-query blocks (8 heads): per block
    # QB k row ids (4 B) and masks (1 B, rounded to 16), plus a count per block
    w64 = L.lib.dsa_sparse_mla_qblocked_workspace_size(4096, 64, 2048)
    w8 = L.lib.dsa_sparse_mla_qblocked_workspace_size(4096, 8, 2048)
    assert w64 >= 1024 * 4 * 2048 * 5 and w64 < 1024 * 4 * 2048 * 5 + (1 << 16)
    assert w8 >= 512 * 8 * 2048 * 5 and w8 < 512 * 8 * 2048 * 5 + (1 << 16)
    assert L.lib.dsa_sparse_mla_qblocked_workspace_size(0, 64, 2048) == 0
    assert L.lib.dsa_sparse_mla_qblocked_workspace_size(4097, 64, 2048) > w64


def test_workspace_sizes_are_pure_functions_of_bounds():
    assert L.lib.dsa_topk_workspace_size(32, 8192, 2048) == 0
    # rows over 32K: keys and positions of k survivors per chunk (16K positions,
    # 32K past 128K)
    assert L.lib.dsa_topk_workspace_size(32, 245760, 2048) == 32 * 8 * 2048 * 8
    assert L.lib.dsa_topk_workspace_size(64, 131072, 2048) == 64 * 8 * 2048 * 8
    s = L.lib.dsa_sparse_mla_workspace_size(32, 64, 512, 2048)
    assert s > 0 and s == L.lib.dsa_sparse_mla_workspace_size(32, 64, 512, 2048)
    assert L.lib.dsa_sparse_mla_workspace_size(4096, 64, 512, 2048) == 0
    assert L.lib.dsa_sparse_mla_workspace_size(0, 64, 512, 2048) == 0


def _append(slots=FAKE, n=4, lat=FAKE, kv=None, keys=FAKE, kd=L.DSA_BF16, kc=None):
    kv = _cache(row_elems=576) if kv is None else kv
    kc = _cache(dtype=L.DSA_FP8_E4M3) if kc is None else kc
    return L.lib.dsa_kv_append(slots, n, lat, ctypes.byref(kv) if kv is not False else None,
                               keys, kd, ctypes.byref(kc) if kc is not False else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), 2),
    (dict(kv=False, kc=False, lat=0, keys=0), 1),
    (dict(lat=0), 1),                                    # latent cache without rows
    (dict(kv=False), 1),                                 # rows without a latent cache
    (dict(keys=0), 1),
    (dict(slots=0), 1),
    (dict(slots=FAKE + 2), 2),                           # misaligned slot mapping
    (dict(kd=L.DSA_FP8_E4M3), 3),                        # keys must arrive as f32 or bf16
    (dict(kc=_cache(dtype=L.DSA_F32), kd=L.DSA_BF16), 3),  # copy needs the cache's type
    (dict(kv=_cache(row_elems=576, dtype=L.DSA_FP8_E4M3)), 3),  # no fp8 latent cache
    (dict(kc=_cache(dtype=L.DSA_FP8_E4M3, scale=0)), 1),
    (dict(kv=_cache(row_elems=576, data=FAKE + 8)), 2),
    (dict(kv=_cache(row_elems=576, page_size=0)), 2),
])
def test_kv_append_rejects_bad_arguments(kw, code):
    assert _append(**kw) == code


def test_kv_append_empty_is_a_no_op():
    assert _append(n=0, slots=0, lat=0, keys=0) == 0


def test_empty_batch_is_a_validated_no_op():
    """total_q = 0: nothing to enqueue, so per-row arrays and the batch's metadata
    may be NULL; the remaining arguments are still checked."""
    b = L.DsaBatch(block_table=None, seq_lens=None, cu_q=None, batch=0, bt_stride=0, total_q=0,
                   max_seq_len=0, max_q=0)
    kc = _cache()
    assert _idx(b=b, q=None, w=None, s=None, ld=1) == 0
    assert _topk(b=b, s=None, idx=None, ld=1) == 0
    assert _mla(b=b, q=None, idx=None, out=None, lse=None, ws=None, wsb=0) == 0
    assert L.lib.dsa_page_scores(ctypes.byref(b), None, 1, 64, None, 1, None) == 0
    assert L.lib.dsa_page_topk(ctypes.byref(b), None, 1, 64, 32, None, None, None, 0, None) == 0
    assert L.lib.dsa_indexer_page_scores(ctypes.byref(b), None, L.DSA_BF16, None, 32, 128,
                                         ctypes.byref(kc), 64, None, 1, None) == 0
    # still validated: strides, k, caches, element types
    assert _idx(b=b, q=None, w=None, s=None, ld=0) == 2
    assert _topk(b=b, s=None, idx=None, ld=1, k=0) == 2
    assert _mla(b=b, c=False, q=None, idx=None, out=None) == 1
    assert _mla(b=b, qd=L.DSA_F32, q=None, idx=None, out=None) == 3
    assert L.lib.dsa_page_topk(ctypes.byref(b), None, 1, 64, 0, None, None, None, 0, None) == 2
    # with queries, the same NULL arrays are errors
    assert _idx(q=None) == 1 and _topk(idx=None) == 1 and _mla(out=None) == 1


def _mla_layers(n=3, b=None, q=True, qd=L.DSA_BF16, caches=None, idx=FAKE, out=True, lse=True,
                ws=FAKE, wsb=1 << 40):
    b = _batch() if b is None else b
    caches = [_cache(row_elems=576) for _ in range(max(n, 1))] if caches is None else caches
    kv = (L.DsaPagedCache * len(caches))(*caches) if caches is not False else None
    arr = lambda: (ctypes.c_void_p * max(n, 1))(*([FAKE] * max(n, 1)))
    qa, oa, la = (arr() if q else None), (arr() if out else None), (arr() if lse else None)
    c = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
    return L.lib.dsa_sparse_mla_fwd_layers(ctypes.byref(b), n, c(qa), qd, 64, 512, 64,
                                           kv, idx, 2048, 0.0625, c(oa), c(la), ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), 2), (dict(n=9), 2),
    (dict(q=False), 1), (dict(out=False), 1), (dict(caches=False), 1), (dict(idx=None), 1),
    (dict(caches=[_cache(row_elems=576), _cache(row_elems=576, page_size=32),
                  _cache(row_elems=576)]), 2),                    # one block table, one page size
    (dict(caches=[_cache(row_elems=576), _cache(row_elems=512), _cache(row_elems=576)]), 2),
    (dict(caches=[_cache(row_elems=576), _cache(row_elems=576, dtype=L.DSA_F32),
                  _cache(row_elems=576)]), 3),
    (dict(ws=None), 4),
])
def test_mla_layers_rejects_bad_arguments(kw, code):
    assert _mla_layers(**kw) == code


def test_mla_layers_workspace_and_empty_batch():
    one = L.lib.dsa_sparse_mla_workspace_size(32, 64, 512, 2048)
    assert L.lib.dsa_sparse_mla_layers_workspace_size(3, 32, 64, 512, 2048) == 3 * one
    assert L.lib.dsa_sparse_mla_layers_workspace_size(0, 32, 64, 512, 2048) == 0
    b = L.DsaBatch(block_table=None, seq_lens=None, cu_q=None, batch=0, bt_stride=0, total_q=0,
                   max_seq_len=0, max_q=0)
    assert _mla_layers(b=b, idx=None, lse=False, ws=None, wsb=0) == 0
