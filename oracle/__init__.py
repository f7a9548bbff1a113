"""CPU oracle for the DSA sparse-attention verify step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path (the HIP library and
its Python binding) never imports this package, and this package never imports
the product path. The arithmetic lives in ``dsa_oracle.c`` (plain C, float64);
this module only marshals numpy arrays through ctypes.

Every function cites the page passage it follows; see the C source header for
the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.dsa_oracle_fp8_decode.argtypes = [ctypes.c_uint8]
        lib.dsa_oracle_fp8_decode.restype = ctypes.c_double
        lib.dsa_oracle_fp8_encode.argtypes = [ctypes.c_float]
        lib.dsa_oracle_fp8_encode.restype = ctypes.c_uint8
        lib.dsa_oracle_fwht_f32.argtypes = [P, i32]
        lib.dsa_oracle_fwht_f32.restype = None
        lib.dsa_oracle_quantize.argtypes = [P, i64, i32, P, P]
        lib.dsa_oracle_quantize.restype = i32
        lib.dsa_oracle_row_visible.argtypes = [P, P, i32, i64]
        lib.dsa_oracle_row_visible.restype = i64
        lib.dsa_oracle_index_score_rows.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, P, i64, P, i64]
        lib.dsa_oracle_index_score_rows.restype = i32
        lib.dsa_oracle_topk.argtypes = [P, i64, P, i64, i32, P]
        lib.dsa_oracle_topk.restype = i32
        lib.dsa_oracle_sparse_mla_rows.argtypes = [P, P, P, i32, P, P, P, P, i32, i32, f32, P, i64, P, P]
        lib.dsa_oracle_sparse_mla_rows.restype = i32
        lib.dsa_oracle_mla_fp8_pack.argtypes = [P, i64, P]
        lib.dsa_oracle_mla_fp8_pack.restype = None
        lib.dsa_oracle_sparse_mla_fp8_rows.argtypes = [P, P, P, i32, P, P, P, P, i32, i32, f32, P, i64,
                                                      P, P]
        lib.dsa_oracle_sparse_mla_fp8_rows.restype = i32
        lib.dsa_oracle_greedy_accept.argtypes = [P, i32, i64, P, i32, i32, i32, P, P, P]
        lib.dsa_oracle_greedy_accept.restype = i32
        lib.dsa_oracle_rejection_accept.argtypes = [P, i32, i64, P, P, P, P, i32, i32, i32, P, P,
                                                    P, P]
        lib.dsa_oracle_rejection_accept.restype = i32
        _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


# ---------------------------------------------------------------------------
# FP8 e4m3fn ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", 配置体系:
# the indexer K cache stores float8_e4m3fn with a per-token fp32 scale).
# ---------------------------------------------------------------------------
def fp8_decode(codes) -> np.ndarray:
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.dsa_oracle_fp8_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def fp8_encode(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.fromiter((lib.dsa_oracle_fp8_encode(float(v)) for v in flat), dtype=np.uint8,
                      count=flat.size)
    return out.reshape(x.shape)


def fwht_f32(x) -> np.ndarray:
    """Sylvester-order fast Walsh-Hadamard transform of each last-axis vector (float32)."""
    lib = _load()
    x = _c(x, np.float32).copy()
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        lib.dsa_oracle_fwht_f32(_p(row), n)
        flat[i] = row
    return flat.reshape(x.shape)


def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """Hadamard rotation + block FP8 quantisation of each last-axis vector.

    ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析", Indexer 的结构与计算流程: q and k are
    Hadamard-rotated and dynamically quantised to FP8 with block size 128.)
    Returns (codes uint8 [..., D], scale float32 [...]).
    """
    lib = _load()
    x = _c(x, np.float32)
    d = x.shape[-1]
    nvec = x.size // d
    codes = np.empty(x.shape, dtype=np.uint8)
    scale = np.empty(x.shape[:-1], dtype=np.float32)
    rc = lib.dsa_oracle_quantize(_p(x), nvec, d, _p(codes), _p(scale))
    if rc != 0:
        raise ValueError(f"oracle quantize: unsupported dim {d}")
    return codes, scale


def row_visible(q_row_offsets, kv_row_offsets, t: int) -> int:
    lib = _load()
    qo = _c(q_row_offsets, np.int32)
    ko = _c(kv_row_offsets, np.int64)
    return int(lib.dsa_oracle_row_visible(_p(qo), _p(ko), len(qo) - 1, t))


def index_score(q_fp8, q_scale, w, k_fp8, k_scale, q_row_offsets, kv_row_offsets,
                rows=None, width=None) -> np.ndarray:
    """Canonical float64 lightning-indexer scores for the given rows.

    Returns [len(rows), width] with -inf beyond each row's visible keys.
    """
    lib = _load()
    q_fp8 = _c(q_fp8, np.uint8)
    T, H, D = q_fp8.shape
    qo = _c(q_row_offsets, np.int32)
    ko = _c(kv_row_offsets, np.int64)
    B = len(qo) - 1
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = _c(rows, np.int64)
    if width is None:
        width = int(np.max(ko[1:] - ko[:-1])) if B else 0
    out = np.empty((len(rows), width), dtype=np.float64)
    rc = lib.dsa_oracle_index_score_rows(
        _p(q_fp8), _p(_c(q_scale, np.float32)), _p(_c(w, np.float32)), _p(_c(k_fp8, np.uint8)),
        _p(_c(k_scale, np.float32)), _p(qo), _p(ko), B, H, D, _p(rows), len(rows), _p(out), width)
    if rc != 0:
        raise ValueError("oracle index_score: a row is outside every request")
    return out


def topk(scores, n_visible, k: int) -> np.ndarray:
    """Top-k positions per row by (score desc, position asc), emitted ascending, -1 padded."""
    lib = _load()
    scores = _c(scores, np.float64)
    if scores.ndim == 1:
        scores = scores[None, :]
    nv = _c(np.broadcast_to(np.asarray(n_visible, dtype=np.int64), (scores.shape[0],)), np.int64)
    out = np.empty((scores.shape[0], k), dtype=np.int32)
    rc = lib.dsa_oracle_topk(_p(scores), scores.shape[1], _p(nv), scores.shape[0], k, _p(out))
    if rc != 0:
        raise ValueError("oracle topk: bad visible count")
    return out


def sparse_mla(q_bf16, kv_bf16, topk_idx, q_row_offsets, kv_row_offsets, sm_scale: float,
               rows=None, share_base=None, num_accepted=None) -> tuple[np.ndarray, np.ndarray]:
    """Float64 sparse MLA over the selected latent rows; returns (out [n,H,512], lse [n,H])."""
    lib = _load()
    q = _c(q_bf16, np.uint16)
    kv = _c(kv_bf16, np.uint16)
    tk = _c(topk_idx, np.int32)
    T, H, dq = q.shape
    assert dq == 576 and kv.shape[-1] == 576
    qo = _c(q_row_offsets, np.int32)
    ko = _c(kv_row_offsets, np.int64)
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = _c(rows, np.int64)
    sb = None if share_base is None else _c(share_base, np.int32)
    na = None if num_accepted is None else _c(num_accepted, np.int32)
    out = np.empty((len(rows), H, 512), dtype=np.float64)
    lse = np.empty((len(rows), H), dtype=np.float64)
    rc = lib.dsa_oracle_sparse_mla_rows(_p(q), _p(kv), _p(tk), tk.shape[1], _p(sb), _p(na),
                                        _p(qo), _p(ko), len(qo) - 1, H, float(sm_scale),
                                        _p(rows), len(rows), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle sparse_mla: a row is outside every request")
    return out, lse


def mla_fp8_pack(latent_bf16) -> np.ndarray:
    """Pack bf16 latent rows [n, 576] into FP8 cache rows [n, 656] ("GLM-5.3 推理全链路(十四)",
    the draft layer's KV pool: 656 bytes per token per layer, fp8_ds_mla): 512 e4m3fn codes
    in 4 blocks of 128 with a float32 scale each, then the 64 rope values in bf16."""
    lib = _load()
    x = _c(latent_bf16, np.uint16)
    assert x.shape[-1] == 576
    n = x.size // 576
    out = np.empty(x.shape[:-1] + (656,), dtype=np.uint8)
    lib.dsa_oracle_mla_fp8_pack(_p(x), n, _p(out))
    return out


def mla_fp8_values(kv8) -> np.ndarray:
    """The float64 values [n, 576] that packed FP8 rows [n, 656] stand for."""
    kv8 = _c(kv8, np.uint8)
    lat = fp8_decode(kv8[..., :512]) * np.repeat(
        kv8[..., 512:528].copy().view(np.float32).astype(np.float64), 128, axis=-1)
    rope = kv8[..., 528:656].copy().view(np.uint16).astype(np.uint32) << 16
    return np.concatenate([lat, rope.view(np.float32).astype(np.float64)], axis=-1)


def sparse_mla_fp8(q_bf16, kv8, topk_idx, q_row_offsets, kv_row_offsets, sm_scale: float,
                   rows=None, share_base=None, num_accepted=None) -> tuple[np.ndarray, np.ndarray]:
    """Float64 sparse MLA over packed FP8 latent rows kv8 [N, 656] (see mla_fp8_pack)."""
    lib = _load()
    q = _c(q_bf16, np.uint16)
    kv8 = _c(kv8, np.uint8)
    tk = _c(topk_idx, np.int32)
    T, H, dq = q.shape
    assert dq == 576 and kv8.shape[-1] == 656
    qo = _c(q_row_offsets, np.int32)
    ko = _c(kv_row_offsets, np.int64)
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = _c(rows, np.int64)
    sb = None if share_base is None else _c(share_base, np.int32)
    na = None if num_accepted is None else _c(num_accepted, np.int32)
    out = np.empty((len(rows), H, 512), dtype=np.float64)
    lse = np.empty((len(rows), H), dtype=np.float64)
    rc = lib.dsa_oracle_sparse_mla_fp8_rows(_p(q), _p(kv8), _p(tk), tk.shape[1], _p(sb), _p(na),
                                            _p(qo), _p(ko), len(qo) - 1, H, float(sm_scale),
                                            _p(rows), len(rows), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle sparse_mla_fp8: a row is outside every request")
    return out, lse


def greedy_accept(logits, draft, K: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Greedy acceptance; logits float32 or bfloat16-as-uint16 [B*(K+1), V], draft [B, K]."""
    lib = _load()
    logits = np.ascontiguousarray(logits)
    if logits.dtype == np.float32:
        dtype = 0
    elif logits.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("logits must be float32 or bfloat16 bits (uint16)")
    rows, V = logits.shape
    B = rows // (K + 1)
    draft = _c(draft, np.int32).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int32)
    n = np.empty(B, dtype=np.int32)
    nxt = np.empty(B, dtype=np.int32)
    am = np.empty(rows, dtype=np.int32)
    rc = lib.dsa_oracle_greedy_accept(_p(logits), dtype, V, _p(np.ascontiguousarray(draft)), B,
                                      K, V, _p(n), _p(nxt), _p(am))
    if rc != 0:
        raise ValueError("oracle greedy_accept: bad arguments")
    return n, nxt, am.reshape(B, K + 1)


def rejection_accept(logits, draft_probs, draft, u, us, K: int):
    """Rejection-sampling acceptance ("GLM-5.3 推理全链路(十四)", "接受判定:greedy 与
    rejection sampling": keep draft i with probability min(1, p/q); at the first refusal
    draw the step's token from the corrected distribution max(0, p - q)).

    logits float32 or bfloat16-as-uint16 [B*(K+1), V]; draft_probs float32 [B, K, V];
    draft int32 [B, K]; u float32 [B, K] and us float32 [B] uniforms in [0, 1).
    Returns (num_accepted [B], next_token [B], acc_margin [B, K], samp_margin [B]): the
    margins are the relative distance of each accept decision and of the draw from their
    boundaries (a float rounding there could flip them).
    """
    lib = _load()
    logits = np.ascontiguousarray(logits)
    if logits.dtype == np.float32:
        dtype = 0
    elif logits.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("logits must be float32 or bfloat16 bits (uint16)")
    rows, V = logits.shape
    B = rows // (K + 1)
    dp = _c(draft_probs, np.float32).reshape(B, K, V) if K else np.zeros((B, 0, V), np.float32)
    dr = _c(draft, np.int32).reshape(B, K) if K else np.zeros((B, 0), np.int32)
    uu = _c(u, np.float32).reshape(B, K) if K else np.zeros((B, 0), np.float32)
    us = _c(us, np.float32).reshape(B)
    n = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    am = np.zeros((B, max(K, 1)), np.float64)
    sm = np.empty(B, np.float64)
    rc = lib.dsa_oracle_rejection_accept(_p(logits), dtype, V, _p(np.ascontiguousarray(dp)),
                                         _p(np.ascontiguousarray(dr)), _p(np.ascontiguousarray(uu)),
                                         _p(us), B, K, V, _p(n), _p(nxt), _p(am), _p(sm))
    if rc != 0:
        raise ValueError("oracle rejection_accept: bad arguments")
    return n, nxt, am[:, :K], sm
