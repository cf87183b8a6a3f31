"""Build libdsa.so (the C-ABI library) in-tree with hipcc for gfx950.

    python sparse_attention_decode_lightning_amd/build.py

Sources are compiled in parallel into ``_build/`` at the repository root and
linked into ``sparse_attention_decode_lightning_amd/libdsa.so``. The
benchmark's read-stream probe (``include/dsa_bench.h``) is linked on its own
into ``libdsa_bench.so``: it is a measurement helper, not part of the path.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
BENCH_LIB = os.path.join(PKG, "libdsa_bench.so")

SOURCES = ["dsa_api.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "kv_append.hip", "page_select.hip"]
BENCH_SOURCES = ["bench_read.hip"]
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source extras: the indexer keeps its MFMA accumulators in ordinary
# vector registers (its epilogue reads every accumulator element once, and
# each read out of the accumulation registers costs a move).
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), "-x", "hip", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("unknown target feature", "packed-fp32-ops", "warning generated")
    err = "\n".join(ln for ln in r.stderr.splitlines() if not any(n in ln for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950, link libdsa.so and libdsa_bench.so; returns the
    path of libdsa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in BENCH_SOURCES], BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build()
