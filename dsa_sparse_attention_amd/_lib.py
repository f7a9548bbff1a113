"""ctypes loader of libdsa.so (the HIP library); fails loudly when it is missing."""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "dsa.h")

_lib = None

P = ctypes.c_void_p
I32, I64, F32, SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

class TopkRefine(ctypes.Structure):
    """dsa_topk_refine of include/dsa.h (device pointers, head count and width, error scale,
    optional key-scale table)."""
    _fields_ = [("q_fp8", P), ("q_scale", P), ("w", P), ("k_fp8", P), ("k_scale", P),
                ("H_I", I32), ("D_I", I32), ("err_scale", ctypes.c_double), ("status", P),
                ("k_scale_max", P), ("k_scale_max_len", I64)]


SIGNATURES = {
    "dsa_abi_version": ([], ctypes.c_int),
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_quantize_fp8": ([P, I64, I32, P, P, P], ctypes.c_int),
    "dsa_verify_cache_write": ([P, P, P, I32, I32, P, P, P, P, I32, P, P, P, P], ctypes.c_int),
    "dsa_key_scale_max": ([P, I64, I64, I64, P, P], ctypes.c_int),
    "dsa_index_score": ([P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I64, P, I64, P],
                        ctypes.c_int),
    "dsa_topk": ([P, I64, P, P, I32, I32, I32, I64, I32, P, P, P, SZ, P], ctypes.c_int),
    "dsa_topk_workspace_size": ([I32, I32, I64, I32, I32], SZ),
    "dsa_index_topk": ([P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I64, I32, ctypes.c_double,
                        P, P, P, P, SZ, P], ctypes.c_int),
    "dsa_index_topk_workspace_size": ([I32, I32, I32, I32, I64], SZ),
    "dsa_sparse_mla_decode": ([P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, F32, P, P, P, SZ, P],
                              ctypes.c_int),
    "dsa_sparse_mla_workspace_size": ([I32, I32, I32], SZ),
    "dsa_sparse_mla_decode_fp8": ([P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, F32, P, P, P, SZ,
                                   P], ctypes.c_int),
    "dsa_mla_fp8_pack": ([P, P, I64, P, P], ctypes.c_int),
    "greedy_accept": ([P, I32, I64, P, I32, I32, I32, P, P, P, P, SZ, P], ctypes.c_int),
    "greedy_accept_workspace_size": ([I32, I32, I32], SZ),
    "greedy_accept_noalloc": ([P, I32, I64, P, I32, I32, I32, P, P, P, P], ctypes.c_int),
    "rejection_accept": ([P, I32, I64, P, P, P, P, I32, I32, I32, P, P, P, SZ, P], ctypes.c_int),
    "rejection_accept_workspace_size": ([I32, I32, I32], SZ),
}


def header_symbols() -> list[str]:
    """Function names declared in include/dsa.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b(\w+)\s*\(", text, re.M)))


def load():
    """Load libdsa.so once; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m dsa_sparse_attention_amd.build). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib
