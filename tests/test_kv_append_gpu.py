"""GPU parity of dsa_kv_append against the oracle: bit-exact bytes and scales.

Small pools (several pages, a ragged set of slots, skipped and out-of-pool
slots) and the real row widths (576-element latent rows, 128-element keys),
with key rows built to hit the e4m3 edge cases: exact midpoints between codes
(ties to even), the subnormal range, the clamp at 448, an all-zero row
(scale 1) and signed zeros.
"""

import zlib

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_decode_lightning_amd as dsa
    return dsa


def _edge_key_rows(rng, D):
    tab = O.e4m3fn_table()
    mags = np.sort(tab[:0x7F])
    mids = (mags[:-1] + mags[1:]) / 2
    rows = []
    # sigma = 448 / 448 = 1 exactly: the row's elements are encoded as given
    r = rng.choice(mids, D).astype(np.float32) * rng.choice([-1, 1], D).astype(np.float32)
    r[0] = 448.0
    rows.append(r)
    r = rng.choice(mags[:16], D).astype(np.float32)  # subnormal range and its midpoints
    r[: D // 2] = rng.choice(mids[:16], D // 2)
    r[1] = -448.0
    rows.append(r)
    rows.append(np.zeros(D, np.float32))  # all zero: scale 1, codes 0
    r = np.zeros(D, np.float32)
    r[::2] = -0.0
    r[3] = 5.0
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("lat_dt", ["bf16", "f32"])
@pytest.mark.parametrize("key_cache_dt,key_src_dt", [("bf16", "bf16"), ("f32", "f32"),
                                                     ("fp8", "bf16"), ("fp8", "f32")])
def test_kv_append_matches_oracle(lat_dt, key_cache_dt, key_src_dt):
    dsa = _dsa()
    dev = torch.device("cuda:0")
    # a seed fixed by the parameters (Python's str hash is salted per process)
    seed = zlib.crc32("|".join((lat_dt, key_cache_dt, key_src_dt)).encode())
    print(f"[kv-append] {lat_dt} {key_cache_dt} {key_src_dt} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    pages, P, R, D = 13, 16, 576, 128
    n_slots = pages * P
    # old cache contents: arbitrary finite values
    lat_np = {"bf16": np.uint16, "f32": np.float32}[lat_dt]
    if lat_dt == "bf16":
        kv_old = (rng.standard_normal((pages, P, R)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    else:
        kv_old = rng.standard_normal((pages, P, R)).astype(np.float32)
    if key_cache_dt == "fp8":
        key_old = rng.integers(0, 0x7F, (pages, P, D), dtype=np.uint8)
        scale_old = rng.random((pages, P)).astype(np.float32)
    elif key_cache_dt == "bf16":
        key_old = (rng.standard_normal((pages, P, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        scale_old = None
    else:
        key_old = rng.standard_normal((pages, P, D)).astype(np.float32)
        scale_old = None
    # 41 tokens: distinct valid slots (ragged, not page aligned), plus skipped ones
    valid = rng.permutation(n_slots)[:37]
    slots = np.concatenate([valid[:20], [-1, n_slots, -7, n_slots + 100], valid[20:]]).astype(np.int32)
    n = len(slots)
    lat_new = (rng.standard_normal((n, R)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) \
        if lat_dt == "bf16" else rng.standard_normal((n, R)).astype(np.float32)
    keys_f = (rng.standard_normal((n, D)) * rng.choice([1e-3, 1.0, 30.0], (n, 1))).astype(np.float32)
    keys_f[: 4] = _edge_key_rows(rng, D)
    if key_src_dt == "bf16":
        keys_new = (keys_f.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16 bits
    else:
        keys_new = keys_f
    ref_kv, ref_key, ref_scale = O.kv_append(slots, lat_new, kv_old, keys_new, key_old, scale_old,
                                             key_cache_dtype=key_cache_dt)

    def t(a, torch_dt=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            x = x.view(torch.int16).view(torch.bfloat16)
        return x.to(dev)

    kv_d = t(kv_old)
    key_d = t(key_old)
    sc_d = t(scale_old) if scale_old is not None else None
    kv_cache = dsa.PagedCache(kv_d)
    k_cache = dsa.PagedCache(key_d, sc_d)
    dsa.kv_append(t(slots), t(lat_new), kv_cache, t(keys_new), k_cache)
    torch.cuda.synchronize()

    def raw(x):
        x = x.cpu()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16)
        return x.numpy()

    assert np.array_equal(raw(kv_d).view(np.uint8), ref_kv.view(np.uint8))
    got_key = raw(key_d)
    assert np.array_equal(got_key.view(np.uint8), ref_key.view(np.uint8)), \
        f"{int((got_key != ref_key).sum())} key elements differ"
    if sc_d is not None:
        assert np.array_equal(raw(sc_d).view(np.uint32), ref_scale.view(np.uint32))


def test_kv_append_empty_and_latent_only():
    dsa = _dsa()
    dev = torch.device("cuda:0")
    kv = torch.randn((4, 8, 576), device=dev).to(torch.bfloat16)
    before = kv.clone()
    dsa.kv_append(torch.empty(0, dtype=torch.int32, device=dev),
                  torch.empty((0, 576), dtype=torch.bfloat16, device=dev), dsa.PagedCache(kv))
    torch.cuda.synchronize()
    assert torch.equal(kv, before)
    rows = torch.randn((3, 576), device=dev).to(torch.bfloat16)
    dsa.kv_append(torch.tensor([5, 31, 0], dtype=torch.int32, device=dev), rows, dsa.PagedCache(kv))
    torch.cuda.synchronize()
    flat, bflat = kv.view(32, 576), before.view(32, 576)
    assert torch.equal(flat[5], rows[0]) and torch.equal(flat[31], rows[1]) and torch.equal(flat[0], rows[2])
    others = [i for i in range(32) if i not in (5, 31, 0)]
    assert torch.equal(flat[others], bflat[others])


def test_kv_append_rejects_bad_arguments():
    dsa = _dsa()
    dev = torch.device("cuda:0")
    kv = dsa.PagedCache(torch.zeros((2, 4, 576), dtype=torch.bfloat16, device=dev))
    fp8 = dsa.PagedCache(torch.zeros((2, 4, 128), dtype=torch.uint8, device=dev),
                         torch.ones((2, 4), device=dev))
    slots = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(TypeError):  # latent rows of the wrong type
        dsa.kv_append(slots, torch.zeros((1, 576), device=dev), kv)
    with pytest.raises(dsa.DSAError):  # fp8 keys must come from f32 or bf16 rows
        bad = torch.zeros((1, 128), dtype=torch.float16, device=dev)
        from sparse_attention_decode_lightning_amd._lib import lib
        import ctypes
        kc = fp8.c()
        dsa.check(lib.dsa_kv_append(slots.data_ptr(), 1, 0, None, bad.data_ptr(), 7,
                                    ctypes.byref(kc), 0), "dsa_kv_append")
