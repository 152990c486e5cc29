"""Thin Python binding of libhils (ctypes over the C ABI in include/hils.h).

Argument marshalling only: every step of the operator runs in the library's
HIP kernels.  Tensors are torch tensors on the current HIP device; the
library call is enqueued on torch's current stream.  If the built library is
missing this module raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhils.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libhils.so not found at {LIB_PATH}; build it with "
                      f"`python -m long_context_landmark_amd.build` (or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)
_i64, _f, _vp, _int, _sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t

_lib.hils_last_error.restype = ctypes.c_char_p
_lib.hils_version.restype = _int
_lib.hils_workspace_size.argtypes = [_int, _i64, _i64, _i64, _i64, _i64, _i64]
_lib.hils_workspace_size.restype = _sz
_lib.hils_landmark_scores.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f, _int, _vp]
_lib.hils_topk_select.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f, _int, _vp, _sz,
                                  _vp]
_lib.hils_sparse_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _f, _int, _vp, _sz, _vp]
_lib.hils_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                  _i64, _f, _int, _vp, _sz, _vp]
_lib.hils_sparse_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                      _i64, _i64, _i64, _i64, _f, _int, _vp, _sz, _vp]
_lib.hils_sparse_attn_fwd_rq.argtypes = [_vp] + _lib.hils_sparse_attn_fwd.argtypes
_lib.hils_decode_step_rq.argtypes = [_vp] + _lib.hils_decode_step.argtypes
_lib.hils_sparse_attn_bwd_rq.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                         _i64, _i64, _i64, _i64, _i64, _f, _int, _vp, _sz, _vp]
_lib.hils_chunk_means.argtypes = [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int, _vp]
_lib.hils_sparse_attn_fwd_lf.argtypes = _lib.hils_sparse_attn_fwd_rq.argtypes
_lib.hils_decode_step_lf.argtypes = _lib.hils_decode_step_rq.argtypes
_lib.hils_decode_step_ml.argtypes = _lib.hils_decode_step_rq.argtypes[:7] + [_i64] + _lib.hils_decode_step_rq.argtypes[7:]
_lib.hils_sparse_attn_bwd_lf.argtypes = _lib.hils_sparse_attn_bwd_rq.argtypes
_lib.hils_sparse_attn_fwd_ml.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64] + _lib.hils_sparse_attn_fwd.argtypes[4:]
_lib.hils_sparse_attn_bwd_ml.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64] + _lib.hils_sparse_attn_bwd_rq.argtypes[5:]
_lib.hils_decode_step_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _int, _vp, _vp,
                                        _vp, _i64, _i64, _i64, _i64, _i64, _f, _int, _vp, _sz, _vp]
_lib.hils_decode_step_noalloc.argtypes = _lib.hils_decode_step.argtypes[:-3] + [_vp]
_lib.hils_profile_enable.argtypes = [_int]
_lib.hils_profile_enable.restype = None
_lib.hils_profile_read.argtypes = [ctypes.c_char_p, _int, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_long), _int]
_lib.hils_profile_read.restype = _int
for _fn in ("hils_landmark_scores", "hils_topk_select", "hils_sparse_attn_fwd", "hils_decode_step",
            "hils_sparse_attn_bwd"):
    getattr(_lib, _fn).restype = _int

OP_SCORES, OP_TOPK, OP_FWD, OP_DECODE, OP_BWD, OP_FWD_ML = range(6)
WS_FP32 = 256  # OR into an operation code for fp32 inputs
BF16, FP32 = 0, 1

EXPORTS = ("hils_last_error", "hils_version", "hils_workspace_size", "hils_landmark_scores", "hils_topk_select",
           "hils_sparse_attn_fwd", "hils_decode_step", "hils_sparse_attn_bwd", "hils_profile_enable",
           "hils_profile_read")


def profile_enable(on: bool = True):
    """Switch per-kernel HIP-event timing on or off (clears the totals)."""
    _lib.hils_profile_enable(1 if on else 0)


def profile_read(max_kernels: int = 64):
    """{kernel name: (total ms, launches)} recorded since profile_enable(True)."""
    stride = 64
    names = ctypes.create_string_buffer(stride * max_kernels)
    ms = (ctypes.c_double * max_kernels)()
    calls = (ctypes.c_long * max_kernels)()
    n = min(_lib.hils_profile_read(names, stride, ms, calls, max_kernels), max_kernels)
    out = {}
    for i in range(n):
        nm = names.raw[i * stride:(i + 1) * stride].split(b"\0", 1)[0].decode()
        out[nm] = (ms[i], calls[i])
    return out


class HilsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libhils status {status}: {msg}")
        self.status = status


def _check(status: int):
    if status != 0:
        raise HilsError(status, _lib.hils_last_error().decode())


def version() -> int:
    return _lib.hils_version()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def workspace_size(op: int, B, H, L, d, C, k) -> int:
    n = _lib.hils_workspace_size(op, B, H, L, d, C, k)
    err = _lib.hils_last_error().decode()
    if n == 0 and err:
        raise HilsError(1, err)
    return n


def _workspace(op, B, H, L, d, C, k, device, ws=None, dtype=None):
    """dtype: the inputs' torch dtype; fp32 inputs keep fp32 per-pair intermediates (a larger workspace)."""
    n = workspace_size(op | (WS_FP32 if dtype == torch.float32 else 0), B, H, L, d, C, k)
    if n == 0:
        return None, 0
    if ws is not None:
        if ws.numel() < n:
            raise ValueError(f"workspace of {ws.numel()} bytes < {n} required")
        return ws, ws.numel()
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _dims(Q, K_lm, C):
    B, H, L, d = Q.shape
    if K_lm.shape != (B, H, L // C, d):
        raise ValueError(f"K_lm must be [B,H,L/C,d] = {(B, H, L // C, d)}, got {tuple(K_lm.shape)}")
    return B, H, L, d


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _like(ret, ref, name):
    if ret is not None and (ret.shape != ref.shape or ret.dtype != ref.dtype or ret.device != ref.device):
        raise ValueError(f"{name} must match the query in shape, dtype and device")


def landmark_scores(Q, K_lm, C=64, scale=None):
    _contig(Q, K_lm)
    B, H, L, d = _dims(Q, K_lm, C)
    S = torch.empty((B, H, L, L // C), dtype=torch.float32, device=Q.device)
    _check(_lib.hils_landmark_scores(_p(Q), _p(K_lm), _p(S), B, H, L, d, C, _scale(d, scale), _dt(Q), _stream()))
    return S


def topk_select(Q, K_lm, k, C=64, scale=None, with_weights=True):
    _contig(Q, K_lm)
    B, H, L, d = _dims(Q, K_lm, C)
    idx = torch.empty((B, H, L, k + 1), dtype=torch.int32, device=Q.device)
    sel = torch.empty((B, H, L, k + 1), dtype=torch.float32, device=Q.device)
    w = torch.empty_like(sel) if with_weights else None
    wsb, n = _workspace(OP_TOPK, B, H, L, d, C, k, Q.device)
    _check(_lib.hils_topk_select(_p(Q), _p(K_lm), _p(idx), _p(sel), _p(w), B, H, L, d, C, k, _scale(d, scale),
                                 _dt(Q), _p(wsb), n, _stream()))
    return idx, sel, w


def sparse_attn_fwd(Q, K, V, K_lm, k, C=64, scale=None, idx=None, save_for_backward=False, ws=None, out=None,
                    Q_ret=None):
    """Returns (O, idx, sel_score, w, lse); w and lse are None unless save_for_backward.

    ``Q_ret``: retrieval queries (Q's shape and dtype) that score the landmarks instead of Q."""
    _contig(Q, K, V, K_lm, idx, Q_ret)
    _like(Q_ret, Q, "Q_ret")
    B, H, L, d = _dims(Q, K_lm, C)
    for t in (K, V):
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError("Q, K, V must share shape and dtype")
    select = 1
    if idx is None:
        idx = torch.empty((B, H, L, k + 1), dtype=torch.int32, device=Q.device)
    else:
        select = 0
        if idx.shape != (B, H, L, k + 1) or idx.dtype != torch.int32:
            raise ValueError("idx must be int32 [B,H,L,k+1]")
    sel = torch.empty((B, H, L, k + 1), dtype=torch.float32, device=Q.device)
    w = torch.empty_like(sel) if save_for_backward else None
    lse = torch.empty_like(sel) if save_for_backward else None
    O = out if out is not None else torch.empty_like(Q)
    wsb, n = _workspace(OP_FWD, B, H, L, d, C, k, Q.device, ws, Q.dtype)
    args = (_p(K), _p(V), _p(K_lm), _p(idx), _p(sel), select, _p(O), _p(w), _p(lse), B, H, L, d, C, k,
            _scale(d, scale), _dt(Q), _p(wsb), n, _stream())
    if Q_ret is None:
        _check(_lib.hils_sparse_attn_fwd(_p(Q), *args))
    else:
        _check(_lib.hils_sparse_attn_fwd_rq(_p(Q), _p(Q_ret), *args))
    return O, idx, sel, w, lse


def chunk_means(K, C=64, n_chunks=None, K_lm=None):
    """Landmark-free chunk keys: rows 0..n_chunks-1 of K_lm [B,H,N_lm,d] become the key means of each chunk of K
    [B,H,L_k,d] (default: every complete chunk, into a new [B,H,L_k//C,d] tensor).  Returns K_lm."""
    _contig(K, K_lm)
    B, H, Lk, d = K.shape
    n_chunks = Lk // C if n_chunks is None else n_chunks
    if K_lm is None:
        K_lm = torch.empty((B, H, Lk // C, d), dtype=K.dtype, device=K.device)
    if K_lm.dtype != K.dtype or K_lm.shape[:2] != (B, H) or K_lm.shape[3] != d:
        raise ValueError("K_lm must be [B,H,N_lm,d] of K's dtype")
    _check(_lib.hils_chunk_means(_p(K), _p(K_lm), B, H, Lk, K_lm.shape[2], n_chunks, d, C, _dt(K), _stream()))
    return K_lm


def sparse_attn_fwd_lf(Q, K, V, k, C=64, scale=None, idx=None, save_for_backward=False, ws=None, out=None,
                       Q_ret=None, K_lm=None):
    """Forward with landmark-free chunks (landmarks = key means, the own chunk's the causal mean).
    Returns (O, idx, sel_score, w, lse, K_lm); K_lm holds the chunks' key means."""
    _contig(Q, K, V, idx, Q_ret, K_lm)
    _like(Q_ret, Q, "Q_ret")
    B, H, L, d = Q.shape
    if L % C:
        raise ValueError("L must be a multiple of C")
    for t in (K, V):
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError("Q, K, V must share shape and dtype")
    K_lm = K_lm if K_lm is not None else torch.empty((B, H, L // C, d), dtype=Q.dtype, device=Q.device)
    if K_lm.shape != (B, H, L // C, d) or K_lm.dtype != Q.dtype:
        raise ValueError("K_lm must be [B,H,L/C,d] of Q's dtype")
    select = 1
    if idx is None:
        idx = torch.empty((B, H, L, k + 1), dtype=torch.int32, device=Q.device)
    else:
        select = 0
        if idx.shape != (B, H, L, k + 1) or idx.dtype != torch.int32:
            raise ValueError("idx must be int32 [B,H,L,k+1]")
    sel = torch.empty((B, H, L, k + 1), dtype=torch.float32, device=Q.device)
    w = torch.empty_like(sel) if save_for_backward else None
    lse = torch.empty_like(sel) if save_for_backward else None
    O = out if out is not None else torch.empty_like(Q)
    wsb, n = _workspace(OP_FWD, B, H, L, d, C, k, Q.device, ws, Q.dtype)
    _check(_lib.hils_sparse_attn_fwd_lf(_p(Q), _p(Q_ret), _p(K), _p(V), _p(K_lm), _p(idx), _p(sel), select, _p(O),
                                        _p(w), _p(lse), B, H, L, d, C, k, _scale(d, scale), _dt(Q), _p(wsb), n,
                                        _stream()))
    return O, idx, sel, w, lse, K_lm


def decode_step(q, k_new, v_new, K_cache, V_cache, K_lm_cache, n_ctx, k, C=64, scale=None, ws=None, out=None,
                idx=None, w=None, q_ret=None, landmark_free=False):
    """One decode step at position n_ctx; returns (o, idx, w).  The caches are updated in place.
    ``q_ret``: retrieval query (q's shape and dtype) that scores the landmarks instead of q.
    ``landmark_free``: the step writes landmark row n_ctx // C of K_lm_cache (the mean of the open chunk's
    keys so far); earlier rows must hold their chunks' key means."""
    _contig(q, k_new, v_new, K_cache, V_cache, K_lm_cache, q_ret)
    _like(q_ret, q, "q_ret")
    B, H, d = q.shape
    L_max = K_cache.shape[2]
    o = out if out is not None else torch.empty_like(q)
    idx = idx if idx is not None else torch.empty((B, H, k + 1), dtype=torch.int32, device=q.device)
    w = w if w is not None else torch.empty((B, H, k + 1), dtype=torch.float32, device=q.device)
    wsb, n = _workspace(OP_DECODE, B, H, L_max, d, C, k, q.device, ws)
    args = (_p(k_new), _p(v_new), _p(K_cache), _p(V_cache), _p(K_lm_cache), n_ctx, L_max, _p(o), _p(idx), _p(w), B,
            H, d, C, k, _scale(d, scale), _dt(q), _p(wsb), n, _stream())
    if K_lm_cache.dim() == 5:
        # several landmarks per chunk: K_lm_cache [B,H,N_max,m,d]
        if landmark_free:
            raise ValueError("landmark-free decode takes one landmark per chunk")
        a = list(args)
        _check(_lib.hils_decode_step_ml(_p(q), _p(q_ret), *a[:5], K_lm_cache.shape[3], *a[5:]))
    elif landmark_free:
        _check(_lib.hils_decode_step_lf(_p(q), _p(q_ret), *args))
    elif q_ret is None:
        _check(_lib.hils_decode_step(_p(q), *args))
    else:
        _check(_lib.hils_decode_step_rq(_p(q), _p(q_ret), *args))
    return o, idx, w


def decode_step_noalloc(q, k_new, v_new, K_cache, V_cache, K_lm_cache, n_ctx, k, C=64, scale=None, out=None,
                        idx=None, w=None):
    """As ``decode_step`` (one landmark per chunk, no retrieval query), without a workspace: the library's
    fixed per-device scratch array holds the step's temporaries (calls on one GPU must not overlap)."""
    _contig(q, k_new, v_new, K_cache, V_cache, K_lm_cache)
    B, H, d = q.shape
    L_max = K_cache.shape[2]
    o = out if out is not None else torch.empty_like(q)
    idx = idx if idx is not None else torch.empty((B, H, k + 1), dtype=torch.int32, device=q.device)
    w = w if w is not None else torch.empty((B, H, k + 1), dtype=torch.float32, device=q.device)
    _check(_lib.hils_decode_step_noalloc(_p(q), _p(k_new), _p(v_new), _p(K_cache), _p(V_cache), _p(K_lm_cache),
                                         n_ctx, L_max, _p(o), _p(idx), _p(w), B, H, d, C, k, _scale(d, scale),
                                         _dt(q), _stream()))
    return o, idx, w


def sparse_attn_bwd(Q, K, V, K_lm, dO, idx, w, lse, k, C=64, scale=None, ws=None, out=None, Q_ret=None):
    """Returns (dQ, dK, dV, dK_lm) in float32, selection held fixed.

    With ``Q_ret`` (the forward's retrieval queries) returns (dQ, dQ_ret, dK, dV, dK_lm): dQ_ret
    takes the gradient of the landmark scores and dQ the in-chunk attention terms."""
    _contig(Q, K, V, K_lm, dO, idx, w, lse, Q_ret)
    _like(Q_ret, Q, "Q_ret")
    B, H, L, d = _dims(Q, K_lm, C)
    f32 = dict(dtype=torch.float32, device=Q.device)
    dQr = None
    if out is not None:
        if Q_ret is None:
            dQ, dK, dV, dKlm = out
        else:
            dQ, dQr, dK, dV, dKlm = out
    else:
        dQ = torch.empty((B, H, L, d), **f32)
        dK = torch.empty((B, H, L, d), **f32)
        dV = torch.empty((B, H, L, d), **f32)
        dKlm = torch.empty((B, H, L // C, d), **f32)
        if Q_ret is not None:
            dQr = torch.empty((B, H, L, d), **f32)
    wsb, n = _workspace(OP_BWD, B, H, L, d, C, k, Q.device, ws, Q.dtype)
    tail = (_p(dK), _p(dV), _p(dKlm), B, H, L, d, C, k, _scale(d, scale), _dt(Q), _p(wsb), n, _stream())
    head = (_p(K), _p(V), _p(K_lm), _p(dO), _p(idx), _p(w), _p(lse))
    if Q_ret is None:
        _check(_lib.hils_sparse_attn_bwd(_p(Q), *head, _p(dQ), *tail))
        return dQ, dK, dV, dKlm
    _check(_lib.hils_sparse_attn_bwd_rq(_p(Q), _p(Q_ret), *head, _p(dQ), _p(dQr), *tail))
    return dQ, dQr, dK, dV, dKlm


def sparse_attn_bwd_lf(Q, K, V, K_lm, dO, idx, w, lse, k, C=64, scale=None, ws=None, Q_ret=None):
    """Backward of ``sparse_attn_fwd_lf`` (K_lm: its key means), selection held fixed.  Returns
    (dQ, dK, dV, dK_lm), or (dQ, dQ_ret, dK, dV, dK_lm) with ``Q_ret``; dK carries the landmark paths and
    dK_lm is the past chunks' mean gradient (already inside dK)."""
    _contig(Q, K, V, K_lm, dO, idx, w, lse, Q_ret)
    _like(Q_ret, Q, "Q_ret")
    B, H, L, d = _dims(Q, K_lm, C)
    f32 = dict(dtype=torch.float32, device=Q.device)
    dQ, dK, dV = (torch.empty((B, H, L, d), **f32) for _ in range(3))
    dKlm = torch.empty((B, H, L // C, d), **f32)
    dQr = torch.empty((B, H, L, d), **f32) if Q_ret is not None else None
    wsb, n = _workspace(OP_BWD, B, H, L, d, C, k, Q.device, ws, Q.dtype)
    _check(_lib.hils_sparse_attn_bwd_lf(_p(Q), _p(Q_ret), _p(K), _p(V), _p(K_lm), _p(dO), _p(idx), _p(w), _p(lse),
                                        _p(dQ), _p(dQr), _p(dK), _p(dV), _p(dKlm), B, H, L, d, C, k, _scale(d, scale),
                                        _dt(Q), _p(wsb), n, _stream()))
    if Q_ret is None:
        return dQ, dK, dV, dKlm
    return dQ, dQr, dK, dV, dKlm


def decode_step_paged(q, k_new, v_new, K_pages, V_pages, K_lm_pages, page_table, n_ctx, n_ctx_max, k, C=64,
                      scale=None, ws=None, out=None, idx=None, w=None, q_ret=None, landmark_free=False):
    """One decode step of B sequences at their own positions n_ctx[b] (int64 device tensor [B]; n_ctx_max >= all
    of them) over page pools K_pages / V_pages [P,H,64,d] and K_lm_pages [P,H,d] (or [P,H,m,d]: m landmarks per
    chunk, log-sum-exp chunk scores), page_table int32 [B,max_pages] (device).  Returns (o, idx, w); the pools are
    updated in place."""
    _contig(q, k_new, v_new, K_pages, V_pages, K_lm_pages, page_table, n_ctx, q_ret)
    _like(q_ret, q, "q_ret")
    B, H, d = q.shape
    P = K_pages.shape[0]
    m = K_lm_pages.shape[2] if K_lm_pages.dim() == 4 else 1
    lm_shape = (P, H, m, d) if K_lm_pages.dim() == 4 else (P, H, d)
    if K_pages.shape != (P, H, C, d) or V_pages.shape != K_pages.shape or K_lm_pages.shape != lm_shape:
        raise ValueError("pools must be [P,H,C,d] (keys, values) and [P,H,d] or [P,H,m,d] (landmarks)")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be int32 [B,max_pages]")
    if n_ctx.dtype != torch.int64 or tuple(n_ctx.shape) != (B,):
        raise ValueError("n_ctx must be int64 [B]")
    max_pages = page_table.shape[1]
    o = out if out is not None else torch.empty_like(q)
    idx = idx if idx is not None else torch.empty((B, H, k + 1), dtype=torch.int32, device=q.device)
    w = w if w is not None else torch.empty((B, H, k + 1), dtype=torch.float32, device=q.device)
    wsb, n = _workspace(OP_DECODE, B, H, max_pages * C, d, C, k, q.device, ws)
    _check(_lib.hils_decode_step_paged(_p(q), _p(q_ret), _p(k_new), _p(v_new), _p(K_pages), _p(V_pages),
                                       _p(K_lm_pages), m, _p(page_table), P, max_pages, _p(n_ctx), int(n_ctx_max),
                                       1 if landmark_free else 0, _p(o), _p(idx), _p(w), B, H, d, C, k,
                                       _scale(d, scale), _dt(q), _p(wsb), n, _stream()))
    return o, idx, w


def sparse_attn_fwd_ml(Q, K, V, K_lm, k, C=64, scale=None, idx=None, save_for_backward=False, ws=None, out=None,
                       Q_ret=None):
    """Forward with several landmarks per chunk: K_lm [B,H,N,m,d]; the chunk score is the log-sum-exp of the
    chunk's landmark scores.  Returns (O, idx, sel_score, w, lse) like ``sparse_attn_fwd``."""
    _contig(Q, K, V, K_lm, idx, Q_ret)
    _like(Q_ret, Q, "Q_ret")
    B, H, L, d = Q.shape
    if K_lm.dim() != 5 or K_lm.shape[:3] != (B, H, L // C) or K_lm.shape[4] != d or K_lm.dtype != Q.dtype:
        raise ValueError("K_lm must be [B,H,L/C,m,d] of Q's dtype")
    m = K_lm.shape[3]
    for t in (K, V):
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError("Q, K, V must share shape and dtype")
    select = 1
    if idx is None:
        idx = torch.empty((B, H, L, k + 1), dtype=torch.int32, device=Q.device)
    else:
        select = 0
        if idx.shape != (B, H, L, k + 1) or idx.dtype != torch.int32:
            raise ValueError("idx must be int32 [B,H,L,k+1]")
    sel = torch.empty((B, H, L, k + 1), dtype=torch.float32, device=Q.device)
    w = torch.empty_like(sel) if save_for_backward else None
    lse = torch.empty_like(sel) if save_for_backward else None
    O = out if out is not None else torch.empty_like(Q)
    wsb, n = _workspace(OP_FWD_ML, B, H, L, d, C, k, Q.device, ws, Q.dtype)
    _check(_lib.hils_sparse_attn_fwd_ml(_p(Q), _p(Q_ret), _p(K), _p(V), _p(K_lm), m, _p(idx), _p(sel), select, _p(O),
                                        _p(w), _p(lse), B, H, L, d, C, k, _scale(d, scale), _dt(Q), _p(wsb), n,
                                        _stream()))
    return O, idx, sel, w, lse


def sparse_attn_bwd_ml(Q, K, V, K_lm, dO, idx, w, lse, k, C=64, scale=None, ws=None, Q_ret=None):
    """Backward of ``sparse_attn_fwd_ml`` (K_lm [B,H,N,m,d], m <= 4), selection held fixed.  Returns
    (dQ, dK, dV, dK_lm) or, with ``Q_ret``, (dQ, dQ_ret, dK, dV, dK_lm); dK_lm is [B,H,N,m,d]."""
    _contig(Q, K, V, K_lm, dO, idx, w, lse, Q_ret)
    _like(Q_ret, Q, "Q_ret")
    B, H, L, d = Q.shape
    m = K_lm.shape[3]
    f32 = dict(dtype=torch.float32, device=Q.device)
    dQ, dK, dV = (torch.empty((B, H, L, d), **f32) for _ in range(3))
    dKlm = torch.empty((B, H, L // C, m, d), **f32)
    dQr = torch.empty((B, H, L, d), **f32) if Q_ret is not None else None
    wsb, n = _workspace(OP_BWD, B, H, L, d, C, k, Q.device, ws, Q.dtype)
    _check(_lib.hils_sparse_attn_bwd_ml(_p(Q), _p(Q_ret), _p(K), _p(V), _p(K_lm), m, _p(dO), _p(idx), _p(w), _p(lse),
                                        _p(dQ), _p(dQr), _p(dK), _p(dV), _p(dKlm), B, H, L, d, C, k, _scale(d, scale),
                                        _dt(Q), _p(wsb), n, _stream()))
    if Q_ret is None:
        return dQ, dK, dV, dKlm
    return dQ, dQr, dK, dV, dKlm
