"""Python names of the C ABI in include/dsa.h (argument marshalling only).

Each function checks dtypes/devices/shapes of torch tensors, allocates any
output the caller did not pass (torch provides device memory), and calls the
HIP library on torch's current stream. Every step of the computation runs in
libdsa.so; there is no Python or CPU implementation behind these names.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

DSA_F32, DSA_BF16 = 0, 1
_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED",
           3: "DSA_ERR_WORKSPACE_TOO_SMALL", 4: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def _check(status: int):
    if status != 0:
        msg = _lib.load().dsa_last_error()
        raise DsaError(status, msg.decode() if msg else "")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t, name, shape):
    """Caller-supplied buffers must have exactly the shape the kernels write."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


FP8_ROW_BYTES = 656  # FP8 latent cache row: 512 e4m3fn codes, 4 float32 scales, 64 bf16


def abi_version() -> int:
    return _lib.load().dsa_abi_version()


def quantize_fp8(x: torch.Tensor, out: torch.Tensor | None = None,
                 scale: torch.Tensor | None = None):
    """Hadamard + e4m3fn quantisation of each last-axis vector (dim 64 or 128)."""
    _dev(x, "x", torch.float32)
    d = x.shape[-1]
    nvec = x.numel() // d if d else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(_lib.load().dsa_quantize_fp8(_p(x), nvec, d, _p(out), _p(scale), _stream()))
    return out, scale


KEY_SCALE_CHUNK = 2048  # cache rows per entry of the key-scale table (DSA_KEY_SCALE_CHUNK)


def key_scale_table_len(N: int) -> int:
    return (N + KEY_SCALE_CHUNK - 1) // KEY_SCALE_CHUNK


def key_scale_max(k_scale, out: torch.Tensor | None = None, row_begin: int = 0,
                  row_end: int | None = None):
    """The key-scale table [ceil(N / 2048)] float32: entry c = the largest scale of cache rows
    2048c .. 2048c + 2047 (every chunk that meets [row_begin, row_end) is recomputed)."""
    _dev(k_scale, "k_scale", torch.float32)
    N = k_scale.numel()
    if out is None:
        out = torch.zeros(key_scale_table_len(N), dtype=torch.float32, device=k_scale.device)
    _dev(out, "out", torch.float32)
    _shape(out, "out", (key_scale_table_len(N),))
    _check(_lib.load().dsa_key_scale_max(_p(k_scale), N, row_begin,
                                         N if row_end is None else row_end, _p(out), _stream()))
    return out


def verify_cache_write(k_new, dst_rows, k_cache, k_scale, latent_new=None, kv_cache=None,
                       q=None, q_fp8=None, q_scale=None, k_scale_max=None):
    """The verify rows' new index keys (quantised) and latent rows into the caches at
    dst_rows, and optionally the queries quantised into q_fp8/q_scale, in one launch.
    k_scale_max: the key-scale table (key_scale_max) to keep up to date, or None."""
    _dev(k_new, "k_new", torch.float32)
    _dev(dst_rows, "dst_rows", torch.int64)
    _dev(k_cache, "k_cache", torch.uint8)
    _dev(k_scale, "k_scale", torch.float32)
    T, D = k_new.shape
    if dst_rows.numel() != T or k_cache.shape[-1] != D:
        raise ValueError("dst_rows must hold T rows and k_cache rows must match k_new's width")
    if (latent_new is None) != (kv_cache is None):
        raise ValueError("latent_new and kv_cache go together")
    if latent_new is not None:
        _dev(latent_new, "latent_new", torch.bfloat16)
        _dev(kv_cache, "kv_cache", torch.bfloat16)
        if latent_new.shape != (T, 576) or kv_cache.shape[-1] != 576:
            raise ValueError("latent rows are 576 bf16 wide")
    H = 0
    if q is not None:
        _dev(q, "q", torch.float32)
        if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D:
            raise ValueError("q must be [T, H, D] with k_new's T and D")
        H = q.shape[1]
        if q_fp8 is None:
            q_fp8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
        if q_scale is None:
            q_scale = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        _dev(q_fp8, "q_fp8", torch.uint8)
        _dev(q_scale, "q_scale", torch.float32)
    if k_scale_max is not None:
        _dev(k_scale_max, "k_scale_max", torch.float32)
        _shape(k_scale_max, "k_scale_max", (key_scale_table_len(k_scale.numel()),))
    _check(_lib.load().dsa_verify_cache_write(
        _p(k_new), _p(latent_new), _p(dst_rows), T, D, _p(k_cache), _p(k_scale), _p(kv_cache),
        _p(q), H, _p(q_fp8), _p(q_scale), _p(k_scale_max), _stream()))
    return q_fp8, q_scale


def index_score(q_fp8, q_scale, w, k_fp8, k_scale, q_row_offsets, kv_row_offsets,
                max_q_rows: int, max_kv_len: int, scores: torch.Tensor | None = None):
    """Indexer scores [T, score_ld]; entries past each row's visible prefix are untouched."""
    _dev(q_fp8, "q_fp8", torch.uint8)
    _dev(k_fp8, "k_fp8", torch.uint8)
    for n, t in (("q_scale", q_scale), ("w", w), ("k_scale", k_scale)):
        _dev(t, n, torch.float32)
    _dev(q_row_offsets, "q_row_offsets", torch.int32)
    _dev(kv_row_offsets, "kv_row_offsets", torch.int64)
    T, H, D = q_fp8.shape
    B = q_row_offsets.numel() - 1
    _shape(q_scale, "q_scale", (T, H))
    _shape(w, "w", (T, H))
    if k_fp8.dim() != 2 or k_fp8.shape[1] != D or k_scale.numel() != k_fp8.shape[0]:
        raise ValueError("k_fp8 must be [N, D_I] with one k_scale per key")
    if scores is None:
        ld = (max_kv_len + 3) // 4 * 4
        scores = torch.empty((T, ld), dtype=torch.float32, device=q_fp8.device)
    _dev(scores, "scores", torch.float32)
    if scores.dim() != 2 or scores.shape[0] != T or scores.shape[1] < max_kv_len:
        raise ValueError(f"scores must be [T={T}, >= {max_kv_len}], got {tuple(scores.shape)}")
    _check(_lib.load().dsa_index_score(
        _p(q_fp8), _p(q_scale), _p(w), _p(k_fp8), _p(k_scale), _p(q_row_offsets),
        _p(kv_row_offsets), B, T, max_q_rows, H, D, max_kv_len, _p(scores), scores.shape[1],
        _stream()))
    return scores


def topk(scores, q_row_offsets, kv_row_offsets, max_q_rows: int, max_kv_len: int, k: int,
         out: torch.Tensor | None = None, refine: dict | None = None,
         workspace: torch.Tensor | None = None):
    """Per-row top-k positions [T, k] (ascending, -1 padded).

    refine: the scored FP8 inputs, dict(q_fp8, q_scale, w, k_fp8, k_scale) plus optional
    err_scale (float), status (int32 [T]) and k_scale_max (the key-scale table of
    key_scale_max over k_scale); the selection then follows the exact scores
    (exact-boundary refine, see dsa_topk in include/dsa.h).
    """
    _dev(scores, "scores", torch.float32)
    _dev(q_row_offsets, "q_row_offsets", torch.int32)
    _dev(kv_row_offsets, "kv_row_offsets", torch.int64)
    T = scores.shape[0]
    B = q_row_offsets.numel() - 1
    if scores.dim() != 2 or scores.shape[1] < max_kv_len:
        raise ValueError(f"scores must be [T, >= {max_kv_len}], got {tuple(scores.shape)}")
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    _dev(out, "out", torch.int32)
    _shape(out, "out", (T, k))
    lib = _lib.load()
    rf = None
    if refine is not None:
        _dev(refine["q_fp8"], "q_fp8", torch.uint8)
        _dev(refine["q_scale"], "q_scale", torch.float32)
        _dev(refine["w"], "w", torch.float32)
        _dev(refine["k_fp8"], "k_fp8", torch.uint8)
        _dev(refine["k_scale"], "k_scale", torch.float32)
        q = refine["q_fp8"]
        if q.dim() != 3 or q.shape[0] != T:
            raise ValueError("refine q_fp8 must be [T, H_I, D_I]")
        _shape(refine["q_scale"], "q_scale", q.shape[:2])
        _shape(refine["w"], "w", q.shape[:2])
        st = refine.get("status")
        if st is not None:
            _dev(st, "status", torch.int32)
            _shape(st, "status", (T,))
        ktab = refine.get("k_scale_max")
        if ktab is not None:
            _dev(ktab, "k_scale_max", torch.float32)
            if ktab.dim() != 1 or ktab.numel() < 1:
                raise ValueError("k_scale_max must be a non-empty 1-d table")
        rf = _lib.TopkRefine(_p(q), _p(refine["q_scale"]), _p(refine["w"]), _p(refine["k_fp8"]),
                             _p(refine["k_scale"]), q.shape[1], q.shape[2],
                             float(refine.get("err_scale", 0.0)), _p(st), _p(ktab),
                             0 if ktab is None else ktab.numel())
    wsb = lib.dsa_topk_workspace_size(B, T, max_kv_len, k, 1 if refine is not None else 0)
    ws = workspace
    if ws is None and wsb:
        ws = torch.empty(wsb, dtype=torch.uint8, device=scores.device)
    if ws is not None:
        _dev(ws, "workspace", torch.uint8)
        wsb = ws.numel()
    _check(lib.dsa_topk(_p(scores), scores.shape[1], _p(q_row_offsets), _p(kv_row_offsets), B, T,
                        max_q_rows, max_kv_len, k, ctypes.byref(rf) if rf is not None else None,
                        _p(out), _p(ws), wsb, _stream()))
    return out


def index_topk_workspace_size(B: int, T: int, max_q_rows: int, H_I: int, max_kv_len: int) -> int:
    return int(_lib.load().dsa_index_topk_workspace_size(B, T, max_q_rows, H_I, max_kv_len))


def index_topk(q_fp8, q_scale, w, k_fp8, k_scale, q_row_offsets, kv_row_offsets,
               max_q_rows: int, max_kv_len: int, k: int, out=None, status=None, path=None,
               err_scale: float = 0.0, workspace=None):
    """Fused indexer score + refined top-k (dsa_index_topk): top-k positions [T, k], ascending,
    -1 padded; status / path (int32 [T]) are filled when given."""
    _dev(q_fp8, "q_fp8", torch.uint8)
    _dev(k_fp8, "k_fp8", torch.uint8)
    for n, t in (("q_scale", q_scale), ("w", w), ("k_scale", k_scale)):
        _dev(t, n, torch.float32)
    _dev(q_row_offsets, "q_row_offsets", torch.int32)
    _dev(kv_row_offsets, "kv_row_offsets", torch.int64)
    T, H, D = q_fp8.shape
    B = q_row_offsets.numel() - 1
    _shape(q_scale, "q_scale", (T, H))
    _shape(w, "w", (T, H))
    if k_fp8.dim() != 2 or k_fp8.shape[1] != D or k_scale.numel() != k_fp8.shape[0]:
        raise ValueError("k_fp8 must be [N, D_I] with one k_scale per key")
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=q_fp8.device)
    _dev(out, "out", torch.int32)
    _shape(out, "out", (T, k))
    for n, t in (("status", status), ("path", path)):
        if t is not None:
            _dev(t, n, torch.int32)
            _shape(t, n, (T,))
    lib = _lib.load()
    need = lib.dsa_index_topk_workspace_size(B, T, max_q_rows, H, max_kv_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_fp8.device)
    wsb = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        wsb = workspace.numel()
    _check(lib.dsa_index_topk(_p(q_fp8), _p(q_scale), _p(w), _p(k_fp8), _p(k_scale),
                              _p(q_row_offsets), _p(kv_row_offsets), B, T, max_q_rows, H, D,
                              max_kv_len, k, float(err_scale), _p(status), _p(path), _p(out),
                              _p(workspace), wsb, _stream()))
    return out


def topk_workspace_size(B: int, T: int, max_kv_len: int, k: int, refine: bool = False) -> int:
    return int(_lib.load().dsa_topk_workspace_size(B, T, max_kv_len, k, 1 if refine else 0))


def sparse_mla_workspace_size(T: int, H: int, k: int) -> int:
    return int(_lib.load().dsa_sparse_mla_workspace_size(T, H, k))


def sparse_mla_decode(q, kv, topk_idx, q_row_offsets, kv_row_offsets, max_q_rows: int,
                      sm_scale: float, share_base=None, num_accepted=None, out=None, lse=None,
                      workspace=None, want_lse: bool = True):
    """Sparse MLA over the selected latent rows: (out [T,H,512] bf16, lse [T,H] f32)."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16)
    _dev(topk_idx, "topk", torch.int32)
    _dev(q_row_offsets, "q_row_offsets", torch.int32)
    _dev(kv_row_offsets, "kv_row_offsets", torch.int64)
    if share_base is not None:
        _dev(share_base, "share_base", torch.int32)
        _dev(num_accepted, "num_accepted", torch.int32)
    T, H, dq = q.shape
    if dq != 576 or kv.shape[-1] != 576:
        raise ValueError("latent rows must be 576 wide (512 latent + 64 rope)")
    k = topk_idx.shape[1]
    B = q_row_offsets.numel() - 1
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", torch.bfloat16)
    _shape(out, "out", (T, H, 512))
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", (T, H))
    lib = _lib.load()
    need = lib.dsa_sparse_mla_workspace_size(T, H, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_mla_decode(
        _p(q), _p(kv), _p(topk_idx), topk_idx.shape[0], _p(share_base), _p(num_accepted), _p(q_row_offsets),
        _p(kv_row_offsets), B, T, max_q_rows, H, k, float(sm_scale), _p(out), _p(lse),
        _p(workspace), wsb, _stream()))
    return out, lse


def mla_fp8_pack(latent, kv_fp8=None, dst_rows=None):
    """FP8 latent cache rows [N, 656] u8 from bf16 latent rows [n, 576]: row dst_rows[i]
    (row i without dst_rows) of kv_fp8 packs latent[i]. Returns kv_fp8."""
    _dev(latent, "latent", torch.bfloat16)
    if latent.shape[-1] != 576:
        raise ValueError("latent rows must be 576 wide (512 latent + 64 rope)")
    n = latent.numel() // 576
    if kv_fp8 is None:
        if dst_rows is not None:
            raise ValueError("dst_rows needs the kv_fp8 cache it indexes")
        kv_fp8 = torch.empty(latent.shape[:-1] + (FP8_ROW_BYTES,), dtype=torch.uint8,
                             device=latent.device)
    _dev(kv_fp8, "kv_fp8", torch.uint8)
    if kv_fp8.shape[-1] != FP8_ROW_BYTES:
        raise ValueError(f"kv_fp8 rows must be {FP8_ROW_BYTES} bytes")
    if dst_rows is not None:
        _dev(dst_rows, "dst_rows", torch.int64)
        _shape(dst_rows, "dst_rows", (n,))
    elif kv_fp8.numel() // FP8_ROW_BYTES < n:
        raise ValueError("kv_fp8 holds fewer rows than latent")
    _check(_lib.load().dsa_mla_fp8_pack(_p(latent), _p(dst_rows), n, _p(kv_fp8), _stream()))
    return kv_fp8


def sparse_mla_decode_fp8(q, kv_fp8, topk_idx, q_row_offsets, kv_row_offsets, max_q_rows: int,
                          sm_scale: float, share_base=None, num_accepted=None, out=None, lse=None,
                          workspace=None, want_lse: bool = True):
    """Sparse MLA over an FP8 latent cache [N, 656] u8 (rows of mla_fp8_pack):
    (out [T,H,512] bf16, lse [T,H] f32)."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv_fp8, "kv_fp8", torch.uint8)
    _dev(topk_idx, "topk", torch.int32)
    _dev(q_row_offsets, "q_row_offsets", torch.int32)
    _dev(kv_row_offsets, "kv_row_offsets", torch.int64)
    if share_base is not None:
        _dev(share_base, "share_base", torch.int32)
        _dev(num_accepted, "num_accepted", torch.int32)
    T, H, dq = q.shape
    if dq != 576 or kv_fp8.shape[-1] != FP8_ROW_BYTES:
        raise ValueError(f"q rows must be 576 wide and kv_fp8 rows {FP8_ROW_BYTES} bytes")
    k = topk_idx.shape[1]
    B = q_row_offsets.numel() - 1
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", torch.bfloat16)
    _shape(out, "out", (T, H, 512))
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", (T, H))
    lib = _lib.load()
    need = lib.dsa_sparse_mla_workspace_size(T, H, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_mla_decode_fp8(
        _p(q), _p(kv_fp8), _p(topk_idx), topk_idx.shape[0], _p(share_base), _p(num_accepted),
        _p(q_row_offsets), _p(kv_row_offsets), B, T, max_q_rows, H, k, float(sm_scale), _p(out),
        _p(lse), _p(workspace), wsb, _stream()))
    return out, lse


def greedy_accept(logits, draft, K: int, argmax: bool = True, workspace=None):
    """Greedy acceptance: (num_accepted [B], next_token [B], argmax [B, K+1] or None)."""
    if not isinstance(logits, torch.Tensor) or not logits.is_cuda or not logits.is_contiguous():
        raise TypeError("logits must be a contiguous CUDA tensor")
    if logits.dtype == torch.float32:
        dt = DSA_F32
    elif logits.dtype == torch.bfloat16:
        dt = DSA_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    rows, V = logits.shape
    B = rows // (K + 1)
    if B * (K + 1) != rows:
        raise ValueError("logits rows must be B*(K+1)")
    if K:
        _dev(draft, "draft", torch.int32)
    dev = logits.device
    n = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    am = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if argmax else None
    lib = _lib.load()
    need = lib.greedy_accept_workspace_size(B, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    _check(lib.greedy_accept(_p(logits), dt, V, _p(draft) if K else None, B, K, V, _p(n), _p(nxt),
                             _p(am), _p(workspace), wsb, _stream()))
    return n, nxt, am


NOALLOC_SCRATCH_BYTES = 1 << 20  # DSA_NOALLOC_SCRATCH_BYTES of include/dsa.h


def greedy_accept_noalloc(logits, draft, K: int, num_accepted=None, next_token=None, argmax=None):
    """greedy_accept through the entry point that allocates nothing (fixed device scratch).

    The outputs may be passed in (num_accepted [B], next_token [B], argmax [B, K+1] int32);
    any left out is allocated here by torch, outside the library call.
    """
    if not isinstance(logits, torch.Tensor) or not logits.is_cuda or not logits.is_contiguous():
        raise TypeError("logits must be a contiguous CUDA tensor")
    if logits.dtype == torch.float32:
        dt = DSA_F32
    elif logits.dtype == torch.bfloat16:
        dt = DSA_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    rows, V = logits.shape
    B = rows // (K + 1)
    if B * (K + 1) != rows:
        raise ValueError("logits rows must be B*(K+1)")
    if K:
        _dev(draft, "draft", torch.int32)
        _shape(draft, "draft", (B, K))
    dev = logits.device
    n = num_accepted if num_accepted is not None else torch.empty(B, dtype=torch.int32, device=dev)
    nxt = next_token if next_token is not None else torch.empty(B, dtype=torch.int32, device=dev)
    for name, t, shape in (("num_accepted", n, (B,)), ("next_token", nxt, (B,))):
        _dev(t, name, torch.int32)
        _shape(t, name, shape)
    if argmax is not None:
        _dev(argmax, "argmax", torch.int32)
        _shape(argmax, "argmax", (B, K + 1))
    _check(_lib.load().greedy_accept_noalloc(_p(logits), dt, V, _p(draft) if K else None, B, K, V,
                                             _p(n), _p(nxt), _p(argmax), _stream()))
    return n, nxt, argmax


def rejection_accept(logits, draft_probs, draft, u, us, K: int, workspace=None):
    """Rejection-sampling acceptance: (num_accepted [B], next_token [B])."""
    if not isinstance(logits, torch.Tensor) or not logits.is_cuda or not logits.is_contiguous():
        raise TypeError("logits must be a contiguous CUDA tensor")
    if logits.dtype == torch.float32:
        dt = DSA_F32
    elif logits.dtype == torch.bfloat16:
        dt = DSA_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    rows, V = logits.shape
    B = rows // (K + 1)
    if B * (K + 1) != rows:
        raise ValueError("logits rows must be B*(K+1)")
    _dev(us, "us", torch.float32)
    if K:
        _dev(draft_probs, "draft_probs", torch.float32)
        _dev(draft, "draft", torch.int32)
        _dev(u, "u", torch.float32)
        if draft_probs.numel() != B * K * V or draft.numel() != B * K or u.numel() != B * K:
            raise ValueError("draft_probs [B,K,V], draft [B,K] and u [B,K] must match the logits")
    if us.numel() != B:
        raise ValueError("us must hold B uniforms")
    dev = logits.device
    n = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    lib = _lib.load()
    need = lib.rejection_accept_workspace_size(B, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    _check(lib.rejection_accept(_p(logits), dt, V, _p(draft_probs) if K else None,
                                _p(draft) if K else None, _p(u) if K else None, _p(us), B, K, V,
                                _p(n), _p(nxt), _p(workspace), wsb, _stream()))
    return n, nxt
