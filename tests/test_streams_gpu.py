"""Calls from several host threads on several streams at once. The library keeps
no state between calls and enqueues all of its work on the stream it is given,
so every thread's results equal, bit for bit, those of the same pass run alone
on the default stream (the passes themselves are checked against the oracle in
the parity tests). The cases cover the split MLA (workspace and combine), the
two-phase top-k (chunk and merge workspace) and fp8 keys."""

import threading

import pytest
import torch

from tests import parity as P
from workloads import make_inputs, small_variant, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_decode": small_variant("decode_b32_l8k", batch=8, lens=4096),
    "fp8_verify_long": small_variant("verify_b8_l240k", batch=2, lens=(40000, 9001)),
    "fp8_ragged": small_variant("indexshare_b64", batch=4, lens=(2049, 100, 777, 4096),
                                n_layers=1),
}
REPEATS = 3


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t


def _same(a, b) -> bool:
    sa, ia, oa = a
    sb, ib, ob = b
    if not (torch.equal(_bits(sa), _bits(sb)) and torch.equal(ia, ib)):
        return False
    return all(torch.equal(_bits(x), _bits(y)) and torch.equal(_bits(u), _bits(v))
               for (x, u), (y, v) in zip(oa, ob))


def test_concurrent_streams_and_threads_match_serial():
    dev = torch.device("cuda:0")
    inputs, serial = {}, {}
    for name, wl in CASES.items():
        print(f"[streams] serial {name}", flush=True)
        inputs[name] = to_device(make_inputs(wl), dev)
        s, i, o = P.run_gpu(inputs[name])
        serial[name] = (s.clone(), i.clone(), [(x.clone(), u.clone()) for x, u in o])

    errors, results = [], {}

    def worker(key, name):
        try:
            stream = torch.cuda.Stream(device=dev)
            got = []
            with torch.cuda.stream(stream):
                for _ in range(REPEATS):
                    got.append(P.run_gpu(inputs[name]))
            stream.synchronize()
            results[key] = (name, got)
        except Exception as e:  # reported on the main thread
            errors.append(f"{key}: {e!r}")

    print("[streams] concurrent", flush=True)
    threads = [threading.Thread(target=worker, args=((name, c), name))
               for name in CASES for c in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    assert len(results) == 2 * len(CASES)
    for key, (name, got) in results.items():
        for rep, r in enumerate(got):
            assert _same(r, serial[name]), f"{key} repeat {rep} differs from the serial pass"
