"""Host-code sanitizer run of the C ABI (CPU only, no kernel is launched).

dsa_api.cpp (argument validation and dispatch) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code and linked
with the library's other objects into a separate shared library; the host
check program tests/c/dsa_host_checks.cpp, built with the same sanitizers,
then runs every entry point's rejection paths against it and checks the
kernels' metadata clamping (row_clamp, clamp_page) on malformed lengths,
offsets and page ids. Any sanitizer report fails the run.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_decode_lightning_amd")
ROCM = "/opt/rocm"


def _asan_runtime():
    hits = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                  "libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")) or _asan_runtime() is None,
                    reason="needs ROCm hipcc and the clang sanitizer runtime")
def test_abi_and_clamps_under_asan_ubsan(tmp_path):
    sys.path.insert(0, PKG)
    import build as B  # the package's build script: source list and flags

    hipcc = os.path.join(ROCM, "bin", "hipcc")
    # host-code sanitizers only: each -fsanitize= is scoped to the host pass
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in B.FLAGS if f not in ("-O3",)] + ["-O1", "-g"]
    api_obj = str(tmp_path / "dsa_api_san.o")
    subprocess.run([hipcc, "-x", "hip", *flags, *san, "-c", os.path.join(PKG, "csrc", "dsa_api.cpp"),
                    "-o", api_obj], check=True, capture_output=True, text=True)
    # the kernels' objects as the regular build makes them (built if missing)
    os.makedirs(B.BUILD, exist_ok=True)
    others = []
    for src in B.SOURCES:
        if src == "dsa_api.cpp":
            continue
        obj = os.path.join(B.BUILD, src + ".o")
        if not os.path.exists(obj):
            obj = B._compile(src)
        others.append(obj)
    lib = str(tmp_path / "libdsa_san.so")
    subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan",
                    "-fsanitize=address,undefined", "-o", lib, api_obj, *others],
                   check=True, capture_output=True, text=True)
    # the check program includes the device header, so it is compiled as HIP
    # (its host code sanitized like the library's)
    exe_obj = str(tmp_path / "dsa_host_checks.o")
    subprocess.run([hipcc, "-x", "hip", *flags, *san, "-c",
                    os.path.join(ROOT, "tests", "c", "dsa_host_checks.cpp"), "-o", exe_obj],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "dsa_host_checks")
    subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared-libasan",
                    "-fsanitize=address,undefined", exe_obj, lib, f"-Wl,-rpath,{tmp_path}",
                    f"-Wl,-rpath,{os.path.dirname(_asan_runtime())}", "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
