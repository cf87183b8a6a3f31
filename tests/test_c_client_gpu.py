"""The C ABI without Python: a plain C program (tests/c/dsa_c_client.c, built with
gcc against include/dsa.h and libdsa.so) runs one decode step of the fp32 tiny
workload; its indices, outputs and lse equal those of the Python binding on the
same inputs bit for bit, and the binding's are checked against the oracle in the
parity tests."""

import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import sparse_attention_decode_lightning_amd as dsa
from sparse_attention_decode_lightning_amd import _lib
from tests import parity as P
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plain_c_client_matches_binding():
    print("[c-client] tiny", flush=True)
    wl = WORKLOADS["tiny"]
    inp_h = make_inputs(wl)
    assert inp_h.q_idx.dtype == torch.float32 and inp_h.kv_cache[0].dtype == torch.float32
    B, L, P_ = wl.batch, inp_h.max_seq_len, wl.page_size
    T = inp_h.total_q
    bt = inp_h.block_table[:, : L // P_].contiguous()
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "client")
        pkg = os.path.dirname(_lib.LIB_PATH)
        subprocess.run(["gcc", "-std=c99", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c",
                                                                          "dsa_c_client.c"),
                        "-L/opt/rocm/lib", "-lamdhip64", "-L", pkg, "-ldsa",
                        f"-Wl,-rpath,{pkg}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
        hdr = np.array([B, L, P_, T, wl.idx_heads, wl.idx_dim, wl.topk, wl.mla_heads, wl.d_latent,
                        wl.d_rope, inp_h.k_cache.shape[0]], dtype=np.int32)
        fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        with open(fin, "wb") as f:
            for a in (hdr, bt.numpy(), inp_h.seq_lens.numpy(), inp_h.cu_q.numpy()):
                f.write(np.ascontiguousarray(a, dtype=np.int32).tobytes())
            for a in (inp_h.q_idx, inp_h.w, inp_h.k_cache, inp_h.q_mla[0], inp_h.kv_cache[0]):
                f.write(a.contiguous().numpy().astype(np.float32).tobytes())
            f.write(np.array([wl.scale], dtype=np.float32).tobytes())
        r = subprocess.run([exe, fin, fout], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        raw = np.fromfile(fout, dtype=np.uint8)
    n_idx, n_out, n_lse = T * wl.topk, T * wl.mla_heads * wl.d_latent, T * wl.mla_heads
    c_idx = raw[: 4 * n_idx].view(np.int32)
    c_out = raw[4 * n_idx: 4 * (n_idx + n_out)].view(np.float32)
    c_lse = raw[4 * (n_idx + n_out):].view(np.float32)
    assert c_lse.size == n_lse
    inp = to_device(inp_h, torch.device("cuda:0"))
    _, idx, outs = P.run_gpu(inp, canary=False)
    out, lse = outs[0]
    assert np.array_equal(c_idx, idx.cpu().numpy().ravel())
    assert np.array_equal(c_out, out.cpu().numpy().ravel())
    assert np.array_equal(c_lse, lse.cpu().numpy().ravel())
