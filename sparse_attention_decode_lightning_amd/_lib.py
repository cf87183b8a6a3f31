"""ctypes view of libdsa.so: structs, status codes and raw entry points.

Argument marshalling only; every step of the computation runs in the HIP
library. Importing this module fails loudly if the library was not built.
"""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "dsa.h")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_MLA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/dsa.h
STATUS_NAMES = {
    0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_DTYPE",
    4: "DSA_ERR_WORKSPACE", 5: "DSA_ERR_UNSUPPORTED", 6: "DSA_ERR_LAUNCH",
}


class DsaBatch(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("cu_q", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("bt_stride", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("max_q", ctypes.c_int32),
    ]


class DsaPagedCache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("row_elems", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class DSAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)} ({code})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python sparse_attention_decode_lightning_amd/build.py` (needs ROCm hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                          ctypes.c_float)
    BP, CP = ctypes.POINTER(DsaBatch), ctypes.POINTER(DsaPagedCache)
    lib.dsa_status_str.restype = ctypes.c_char_p
    lib.dsa_status_str.argtypes = [ctypes.c_int]
    lib.dsa_abi_version.restype = I32
    lib.dsa_abi_version.argtypes = []
    lib.dsa_indexer_scores.restype = ctypes.c_int
    lib.dsa_indexer_scores.argtypes = [BP, P, I32, P, I32, I32, CP, P, I64, P]
    lib.dsa_topk_workspace_size.restype = SZ
    lib.dsa_topk_workspace_size.argtypes = [I32, I32, I32]
    lib.dsa_topk.restype = ctypes.c_int
    lib.dsa_topk.argtypes = [BP, P, I64, I32, P, P, SZ, P]
    lib.dsa_sparse_mla_workspace_size.restype = SZ
    lib.dsa_sparse_mla_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.dsa_sparse_mla_fwd.restype = ctypes.c_int
    lib.dsa_sparse_mla_fwd.argtypes = [BP, P, I32, I32, I32, I32, CP, P, I32, F, P, P, P, SZ, P]
    lib.dsa_sparse_mla_fwd_noalloc.restype = ctypes.c_int
    lib.dsa_sparse_mla_fwd_noalloc.argtypes = [BP, P, I32, I32, I32, I32, CP, P, I32, F, P, P, P]
    lib.dsa_sparse_mla_qblocked_workspace_size.restype = SZ
    lib.dsa_sparse_mla_qblocked_workspace_size.argtypes = [I32, I32, I32]
    lib.dsa_sparse_mla_fwd_qblocked.restype = ctypes.c_int
    lib.dsa_sparse_mla_fwd_qblocked.argtypes = [BP, P, I32, I32, I32, I32, CP, P, I32, F, P, P, P,
                                                SZ, P]
    lib.dsa_sparse_mla_layers_workspace_size.restype = SZ
    lib.dsa_sparse_mla_layers_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.dsa_sparse_mla_fwd_layers.restype = ctypes.c_int
    lib.dsa_sparse_mla_fwd_layers.argtypes = [BP, I32, P, I32, I32, I32, I32, CP, P, I32, F, P, P,
                                              P, SZ, P]
    lib.dsa_indexer_page_scores.restype = ctypes.c_int
    lib.dsa_indexer_page_scores.argtypes = [BP, P, I32, P, I32, I32, CP, I32, P, I64, P]
    lib.dsa_indexer_topk_state_size.restype = SZ
    lib.dsa_indexer_topk_state_size.argtypes = [I32]
    lib.dsa_indexer_topk.restype = ctypes.c_int
    lib.dsa_indexer_topk.argtypes = [BP, P, I32, P, I32, I32, CP, I32, P, I64, P, P, SZ, P]
    lib.dsa_page_scores.restype = ctypes.c_int
    lib.dsa_page_scores.argtypes = [BP, P, I64, I32, P, I64, P]
    lib.dsa_page_topk_workspace_size.restype = SZ
    lib.dsa_page_topk_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.dsa_page_topk.restype = ctypes.c_int
    lib.dsa_page_topk.argtypes = [BP, P, I64, I32, I32, P, P, P, SZ, P]
    lib.dsa_kv_append.restype = ctypes.c_int
    lib.dsa_kv_append.argtypes = [P, I32, P, CP, P, I32, CP, P]
    return lib


lib = _load()


def status_str(code: int) -> str:
    return lib.dsa_status_str(int(code)).decode()


def check(code: int, where: str) -> None:
    if code != 0:
        raise DSAError(code, where)


def declared_functions() -> list:
    """Names of every function the public header declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))
