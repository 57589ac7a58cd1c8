"""Python binding of the MI355X sparse-attention library (libsa_mi355x.so).

Argument marshalling only: every function below takes torch tensors that
already live on the GPU (or, where an entry point allows host placement, in
pinned host memory), checks their dtype/shape/contiguity, and passes raw
pointers, sizes and the current HIP stream to the C entry point of the same
name.  All computation happens in the HIP kernels.  If the shared
library has not been built, importing this package raises ImportError; there
is no CPU fallback.

Build: ``python long_context_sparse_apply_amd/build.py``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsa_mi355x.so")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_DTYPE, SA_ERR_RANGE, SA_ERR_WORKSPACE, \
    SA_ERR_UNSUPPORTED, SA_ERR_HIP, SA_ERR_ACCESS = range(9)
SA_F32, SA_BF16 = 0, 1
SA_OP_BLOCK_SCORE, SA_OP_TOPK, SA_OP_DECODE, SA_OP_TOKEN_TOPK = 1, 2, 3, 4

EXPORTED = ("sa_rope_apply", "sa_kv_cache_append", "sa_block_score", "sa_token_score",
            "sa_token_topk", "sa_topk_select", "sa_prefill_row_params", "sa_sparse_attn_prefill",
            "sa_sparse_attn_decode", "sa_sparse_attn_decode_static",
            "sa_calibrate_dominant", "sa_calibrate_workspace_bytes", "sa_sfa_sparsify",
            "sa_workspace_bytes",
            "sa_status_string", "sa_version")


class SAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python long_context_sparse_apply_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, D, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                           ctypes.c_float, ctypes.c_size_t)
    sig = {
        "sa_rope_apply": [P, P, I, I, I, I, I, P, I, D, P],
        "sa_kv_cache_append": [P, P, I, I, I, I, I, I, P, D, I, P, I, P, P, P, P],
        "sa_block_score": [P, P, I, I, I, I, I, I, D, I, I, I, F, I, P, F, P, P, P, P, P, SZ, P],
        "sa_token_score": [P, P, P, I, I, I, I, I, I, P, P, I, I, F, P, P],
        "sa_token_topk": [P, P, I, I, I, I, I, I, P, P, I, I, F, I, P, I, P, P, SZ, P],
        "sa_topk_select": [P, I64, I, P, P, I, I, I, P, I, P, P, SZ, P],
        "sa_prefill_row_params": [I, I64, I, I, I, P, P],
        "sa_sparse_attn_prefill": [P, P, P, I, I, I, I, I, I, I, P, P, I, I, F, P, P, P],
        "sa_sparse_attn_decode": [P, P, P, P, I, I, I, I, I, I, P, P, I, I, P, P, I, F, P, P, P,
                                  SZ, P],
        "sa_sparse_attn_decode_static": [P, P, P, P, I, I, I, I, I, I, P, P, I, I, P, P, I, F, P,
                                         P, P],
        "sa_calibrate_dominant": [P, P, I, I, I, I, I, I, I, I, P, P, P, SZ, P],
        "sa_calibrate_workspace_bytes": [I, I, I, I, I, I],
        "sa_sfa_sparsify": [P, P, I, I64, I, I, P],
        "sa_workspace_bytes": [I, I64, I, I, I, I],
        "sa_status_string": [I],
        "sa_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I
    lib.sa_workspace_bytes.restype = SZ
    lib.sa_calibrate_workspace_bytes.restype = SZ
    lib.sa_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_string(s: int) -> str:
    return lib.sa_status_string(int(s)).decode()


def workspace_bytes(op: int, rows: int = 0, cols: int = 0, B: int = 0, Hq: int = 0,
                    max_k: int = 0) -> int:
    return int(lib.sa_workspace_bytes(op, rows, cols, B, Hq, max_k))


# ----------------------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype=None, ndim=None, host_ok=False):
    """host_ok: pinned host tensors are accepted too (host placement of the
    non-dominant keys and the values, FASA-M)."""
    if t is None:
        return
    if not t.is_cuda and not (host_ok and t.is_pinned()):
        raise ValueError(f"{name} must be a GPU tensor" + (" or pinned host tensor" if host_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _call(name, *args):
    st = getattr(lib, name)(*args)
    if st != SA_OK:
        raise SAError(name, st)


# ----------------------------------------------------------------------------- entry points
def sa_rope_apply(x, out, theta: float, pos=None, pos0: int = 0, stream=None):
    """x, out: [B, H, S, d]; pos: int32 [B*S] or None (pos0 + s)."""
    torch = _torch()
    _check(x, "x", ndim=4)
    _check(out, "out", x.dtype, 4)
    _check(pos, "pos", torch.int32)
    B, H, S, d = x.shape
    _call("sa_rope_apply", _ptr(x), _ptr(out), _dtype_code(x), B, H, S, d, _ptr(pos), pos0,
          float(theta), _stream(stream))
    return out


def sa_kv_cache_append(k_new, v_new, start, k_cache, v_cache, *, theta: float, k_rest=None,
                       dom_pairs=None, slab: bool = False, full_rows: bool = False,
                       stream=None):
    """Write new tokens into a decode KV cache.

    k_new, v_new: [B, Hkv, S, d] raw keys and values; start: int32 [B], the
    cache row (= absolute position) of each batch's first new token.
    slab False: k_cache [B, Hkv, Lmax, d].  slab True: k_cache = k_dom
    [B, Hkv, Lmax, 2*n_dom], k_rest [B, Hkv, Lmax, d - 2*n_dom], dom_pairs
    int32 [Hkv, n_dom]; with full_rows, k_rest holds the full rotated rows
    [B, Hkv, Lmax, d] instead (the slab + full-row layout).  v_cache
    [B, Hkv, Lmax, d].
    """
    torch = _torch()
    _check(k_new, "k_new", ndim=4)
    _check(v_new, "v_new", k_new.dtype, 4)
    _check(start, "start", torch.int32, 1)
    _check(k_cache, "k_cache", k_new.dtype, 4)
    _check(k_rest, "k_rest", k_new.dtype, 4, host_ok=True)
    _check(v_cache, "v_cache", k_new.dtype, 4, host_ok=True)
    _check(dom_pairs, "dom_pairs", torch.int32, 2)
    B, Hkv, S, d = k_new.shape
    if tuple(v_new.shape) != (B, Hkv, S, d) or start.shape[0] != B:
        raise ValueError("k_new / v_new / start shapes disagree")
    Lmax = v_cache.shape[2]
    if tuple(v_cache.shape) != (B, Hkv, Lmax, d):
        raise ValueError("v_cache must be [B, Hkv, Lmax, d]")
    n_dom = 0
    if slab:
        if dom_pairs is None:
            raise ValueError("slab layout needs dom_pairs")
        n_dom = dom_pairs.shape[1]
        if tuple(k_cache.shape) != (B, Hkv, Lmax, 2 * n_dom):
            raise ValueError("k_dom must be [B, Hkv, Lmax, 2*n_dom]")
        rest_w = d if full_rows else d - 2 * n_dom
        if k_rest is not None and tuple(k_rest.shape) != (B, Hkv, Lmax, rest_w):
            raise ValueError(f"k_rest must be [B, Hkv, Lmax, {rest_w}]")
    elif full_rows:
        raise ValueError("full_rows needs the slab layout")
    elif tuple(k_cache.shape) != (B, Hkv, Lmax, d):
        raise ValueError("k_cache must be [B, Hkv, Lmax, d]")
    layout = 0 if not slab else (2 if full_rows else 1)
    _call("sa_kv_cache_append", _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, Hkv, S, d, Lmax,
          _ptr(start), float(theta), layout, _ptr(dom_pairs), n_dom, _ptr(k_cache),
          _ptr(k_rest), _ptr(v_cache), _stream(stream))


def sa_block_score(q, k, scores, *, theta: float, block: int, band_split_pair: int,
                   calibrate: bool = True, sm_scale: float, causal: bool = True, q_rope_out=None,
                   q_rope_scale: float = 1.0, k_rope_out=None, pooled_q_out=None,
                   pooled_k_out=None, ws=None, stream=None):
    """q [B,Hq,S,d], k [B,Hkv,S,d] (raw) -> scores [B,Hq,N,N] fp32.

    q_rope_out receives the rotated Q times q_rope_scale (rounded to q's dtype).
    """
    torch = _torch()
    _check(q, "q", ndim=4)
    _check(k, "k", q.dtype, 4)
    _check(scores, "scores", torch.float32, 4)
    for t, n in ((q_rope_out, "q_rope_out"), (k_rope_out, "k_rope_out")):
        _check(t, n, q.dtype, 4)
    for t, n in ((pooled_q_out, "pooled_q_out"), (pooled_k_out, "pooled_k_out"), (ws, "ws")):
        _check(t, n)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _call("sa_block_score", _ptr(q), _ptr(k), _dtype_code(q), B, Hq, Hkv, S, d, float(theta),
          block, band_split_pair, int(bool(calibrate)), float(sm_scale), int(bool(causal)),
          _ptr(q_rope_out), float(q_rope_scale), _ptr(k_rope_out), _ptr(pooled_q_out),
          _ptr(pooled_k_out),
          _ptr(scores), _ptr(ws), ws_bytes, _stream(stream))
    return scores


def sa_token_score(q_rope, k, scores, cache_len, dom_pairs, *, sm_scale: float, slab: bool = False,
                   k_rest=None, d=None, stream=None):
    """q_rope [B,Hq,d]; k [B,Hkv,Lmax,d] or k_dom [B,Hkv,Lmax,2*n_dom] -> scores [B,Hq,Lmax]."""
    torch = _torch()
    _check(q_rope, "q_rope", ndim=3)
    _check(k, "k", q_rope.dtype, 4)
    _check(scores, "scores", torch.float32, 3)
    _check(cache_len, "cache_len", torch.int32, 1)
    _check(dom_pairs, "dom_pairs", torch.int32, 2)
    B, Hq, dd = q_rope.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    n_dom = dom_pairs.shape[1]
    _call("sa_token_score", _ptr(q_rope), _ptr(k), _ptr(k_rest), _dtype_code(q_rope), B, Hq, Hkv,
          Lmax, dd, _ptr(cache_len), _ptr(dom_pairs), n_dom, int(bool(slab)), float(sm_scale),
          _ptr(scores), _stream(stream))
    return scores


def sa_token_topk(q_rope, k, cache_len, dom_pairs, idx_out, count_out, ws, *, sm_scale: float,
                  k_top: int, slab: bool = True, stream=None):
    """Token scores from the dominant channels and their top-k per (b, h) row
    in one call, without a score array: q_rope [B,Hq,d], k the slab
    [B,Hkv,Lmax,2*n_dom] (slab=True) or the standard cache [B,Hkv,Lmax,d] ->
    idx_out [B,Hq,max_out] (max_out >= k_top), count_out [B,Hq].  ws: uint8 of
    workspace_bytes(SA_OP_TOKEN_TOPK, rows=B*Hq, cols=Lmax, max_k=k_top)."""
    torch = _torch()
    _check(q_rope, "q_rope", ndim=3)
    _check(k, "k", q_rope.dtype, 4)
    _check(cache_len, "cache_len", torch.int32, 1)
    _check(dom_pairs, "dom_pairs", torch.int32, 2)
    _check(idx_out, "idx_out", torch.int32)
    _check(count_out, "count_out", torch.int32)
    if ws is None:
        raise ValueError("sa_token_topk needs its workspace")
    _check(ws, "ws")
    B, Hq, dd = q_rope.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    n_dom = dom_pairs.shape[1]
    max_out = idx_out.shape[-1]
    if idx_out.numel() != B * Hq * max_out or count_out.numel() != B * Hq:
        raise ValueError("idx_out / count_out do not match the (b, h) rows")
    _call("sa_token_topk", _ptr(q_rope), _ptr(k), _dtype_code(q_rope), B, Hq, Hkv, Lmax, dd,
          _ptr(cache_len), _ptr(dom_pairs), n_dom, 1 if slab else 0, float(sm_scale), int(k_top),
          _ptr(idx_out), max_out, _ptr(count_out), _ptr(ws), ws.numel() * ws.element_size(),
          _stream(stream))
    return idx_out, count_out


def sa_topk_select(scores, idx_out, count_out, *, k_const: int, valid_len=None, k_per_row=None,
                   n_sink: int = 0, n_local: int = 0, ws=None, stream=None):
    """scores [..., cols] fp32 (rows = product of leading dims) -> idx_out [rows, max_out]."""
    torch = _torch()
    _check(scores, "scores", torch.float32)
    _check(idx_out, "idx_out", torch.int32)
    _check(count_out, "count_out", torch.int32)
    _check(valid_len, "valid_len", torch.int32)
    _check(k_per_row, "k_per_row", torch.int32)
    cols = scores.shape[-1]
    rows = scores.numel() // cols
    max_out = idx_out.shape[-1]
    if idx_out.numel() != rows * max_out or count_out.numel() != rows:
        raise ValueError("idx_out / count_out do not match the score rows")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _call("sa_topk_select", _ptr(scores), rows, cols, _ptr(valid_len), _ptr(k_per_row), k_const,
          n_sink, n_local, _ptr(idx_out), max_out, _ptr(count_out), _ptr(ws), ws_bytes,
          _stream(stream))
    return idx_out, count_out


def sa_sparse_attn_prefill(q_rope, k_rope, v, blk_idx, blk_cnt, out, *, block: int, sm_scale: float,
                           causal: bool = True, lse=None, stream=None):
    """q_rope [B,Hq,S,d], k_rope/v [B,Hkv,S,d], blk_idx [B,Hq,N,max_sel] -> out [B,Hq,S,d]."""
    torch = _torch()
    _check(q_rope, "q_rope", ndim=4)
    _check(k_rope, "k_rope", q_rope.dtype, 4)
    _check(v, "v", q_rope.dtype, 4)
    _check(out, "out", q_rope.dtype, 4)
    _check(blk_idx, "blk_idx", torch.int32, 4)
    _check(blk_cnt, "blk_cnt", torch.int32, 3)
    _check(lse, "lse", torch.float32)
    B, Hq, S, d = q_rope.shape
    Hkv = k_rope.shape[1]
    _call("sa_sparse_attn_prefill", _ptr(q_rope), _ptr(k_rope), _ptr(v), _dtype_code(q_rope), B,
          Hq, Hkv, S, d, block, _ptr(blk_idx), _ptr(blk_cnt), blk_idx.shape[-1],
          int(bool(causal)), float(sm_scale), _ptr(out), _ptr(lse), _stream(stream))
    return out


def sa_sparse_attn_decode(q_rope, k, v, tok_idx, tok_cnt, out, ws, *, sm_scale: float,
                          cache_len=None, dom_pairs=None, slab: bool = False, k_rest=None,
                          lse=None, stream=None):
    """q_rope [B,Hq,d]; k (or k_dom) / v caches; tok_idx [B,Hq,max_k] -> out [B,Hq,d]."""
    torch = _torch()
    _check(q_rope, "q_rope", ndim=3)
    _check(k, "k", q_rope.dtype, 4)
    _check(k_rest, "k_rest", q_rope.dtype, 4, host_ok=True)
    _check(v, "v", q_rope.dtype, 4, host_ok=True)
    _check(out, "out", q_rope.dtype, 3)
    _check(tok_idx, "tok_idx", torch.int32, 3)
    _check(tok_cnt, "tok_cnt", torch.int32, 2)
    _check(ws, "ws")
    _check(lse, "lse", torch.float32)
    B, Hq, d = q_rope.shape
    Hkv, Lmax = v.shape[1], v.shape[2]
    n_dom = 0 if dom_pairs is None else dom_pairs.shape[1]
    ws_bytes = ws.numel() * ws.element_size()
    _call("sa_sparse_attn_decode", _ptr(q_rope), _ptr(k), _ptr(k_rest), _ptr(v),
          _dtype_code(q_rope), B, Hq, Hkv, Lmax, d, _ptr(cache_len), _ptr(dom_pairs), n_dom,
          int(bool(slab)), _ptr(tok_idx), _ptr(tok_cnt), tok_idx.shape[-1], float(sm_scale),
          _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))
    return out


def sa_sparse_attn_decode_static(q_rope, k, v, tok_idx, tok_cnt, out, *, sm_scale: float,
                                 cache_len=None, dom_pairs=None, slab: bool = False, k_rest=None,
                                 lse=None, stream=None):
    """sa_sparse_attn_decode without a workspace: the split-K partials live in
    the library's fixed per-GPU array (no allocation; calls that overlap on
    one GPU race)."""
    torch = _torch()
    _check(q_rope, "q_rope", ndim=3)
    _check(k, "k", q_rope.dtype, 4)
    _check(k_rest, "k_rest", q_rope.dtype, 4, host_ok=True)
    _check(v, "v", q_rope.dtype, 4, host_ok=True)
    _check(out, "out", q_rope.dtype, 3)
    _check(tok_idx, "tok_idx", torch.int32, 3)
    _check(tok_cnt, "tok_cnt", torch.int32, 2)
    _check(lse, "lse", torch.float32)
    B, Hq, d = q_rope.shape
    Hkv, Lmax = v.shape[1], v.shape[2]
    n_dom = 0 if dom_pairs is None else dom_pairs.shape[1]
    _call("sa_sparse_attn_decode_static", _ptr(q_rope), _ptr(k), _ptr(k_rest), _ptr(v),
          _dtype_code(q_rope), B, Hq, Hkv, Lmax, d, _ptr(cache_len), _ptr(dom_pairs), n_dom,
          int(bool(slab)), _ptr(tok_idx), _ptr(tok_cnt), tok_idx.shape[-1], float(sm_scale),
          _ptr(out), _ptr(lse), _stream(stream))
    return out


def calibrate_workspace_bytes(Hq: int, Hkv: int, M: int, L: int, d: int, k_cal: int) -> int:
    return int(lib.sa_calibrate_workspace_bytes(Hq, Hkv, M, L, d, k_cal))


def sa_calibrate_dominant(q_rope, k_rope, dom_out, counts_out, ws, *, k_cal: int, stream=None):
    """q_rope [Hq, M, d], k_rope [Hkv, L, d] (bf16, rotated) -> dom_out [Hkv, n_dom],
    counts_out [Hkv, d/2] (int32): the offline calibration of the dominant pairs."""
    torch = _torch()
    _check(q_rope, "q_rope", ndim=3)
    _check(k_rope, "k_rope", q_rope.dtype, 3)
    _check(dom_out, "dom_out", torch.int32, 2)
    _check(counts_out, "counts_out", torch.int32, 2)
    _check(ws, "ws")
    Hq, M, d = q_rope.shape
    Hkv, L = k_rope.shape[0], k_rope.shape[1]
    if k_rope.shape[2] != d or dom_out.shape[0] != Hkv or tuple(counts_out.shape) != (Hkv, d // 2):
        raise ValueError("q_rope / k_rope / dom_out / counts_out shapes disagree")
    _call("sa_calibrate_dominant", _ptr(q_rope), _ptr(k_rope), _dtype_code(q_rope), Hq, Hkv, M, L,
          d, int(k_cal), dom_out.shape[1], _ptr(dom_out), _ptr(counts_out), _ptr(ws),
          ws.numel() * ws.element_size(), _stream(stream))
    return dom_out, counts_out


def sa_sfa_sparsify(x, out, *, k_feat: int, stream=None):
    """x, out [..., d] (out may be x): k-sparse feature codes of every row."""
    _check(x, "x")
    _check(out, "out", x.dtype)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    d = x.shape[-1]
    _call("sa_sfa_sparsify", _ptr(x), _ptr(out), _dtype_code(x), x.numel() // d, d, int(k_feat),
          _stream(stream))
    return out


# ----------------------------------------------------------------------------- setup helpers
def prefill_row_params(B: int, Hq: int, N: int, *, keep_const: int = 0, keep_percent: int = 0,
                       causal: bool = True, device="cuda"):
    """Per-row arguments of sa_topk_select for the B*Hq*N prefill block rows,
    from the library's sa_prefill_row_params (the keep budget lives in the C
    library).  Returns (valid_len, k_per_row, k_max) with int32 tensors of
    B*Hq*N entries on ``device``; built once per shape."""
    import numpy as np
    torch = _torch()
    rows = B * Hq * N
    vl = np.empty(rows, np.int32)
    kr = np.empty(rows, np.int32)
    kmax = lib.sa_prefill_row_params(int(N), int(B * Hq), 1 if causal else 0, int(keep_const),
                                     int(keep_percent), vl.ctypes.data_as(ctypes.c_void_p),
                                     kr.ctypes.data_as(ctypes.c_void_p))
    if kmax < 0:
        raise SAError("sa_prefill_row_params", -kmax)
    return torch.from_numpy(vl).to(device), torch.from_numpy(kr).to(device), int(kmax)
