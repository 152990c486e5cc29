"""CPU oracle for HiLS attention (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls anything here.

The arithmetic lives in ``hils_oracle.c`` (plain C, double precision; see its
header for the passages of the HiLS pages each step follows).  This module only
marshals numpy arrays through ctypes.  Inputs are either ``float32`` arrays or
``uint16`` arrays holding bf16 bit patterns.

Parity status of each function (what pins it is in ``tests/test_oracle_*.py``):
  landmark_scores  pinned (numpy einsum in fp64)
  landmark_scores_rows  pinned (rows of the einsum scores in the order listed, and equal
                   to the same rows of landmark_scores)
  fwd (selection)  pinned (numpy lexsort, subset brute force, exact ties)
  fwd (attention)  pinned (dense causal attention via the chunk-LSE identity,
                   single-chunk reduction, equal-score mean, invariances)
  decode           pinned (single-chunk reduction; prefill-row consistency)
  bwd              pinned (central finite differences, closed-form sums)
  retrieval query  pinned (Q_ret = Q reproduces the plain operator; selection depends on
                   Q_ret only; finite differences of dQ_ret, dQ and dKlm)
  landmark-free    pinned (key means against numpy; rows ending a chunk equal the plain
                   operator on numpy means; own score of a chunk's first row is the scaled
                   q.k; own score against numpy prefix means; decode steps equal prefill rows)
  fwd_ml, bwd_ml   pinned (one landmark per chunk is the plain operator bit for bit;
  (several         duplicated landmarks shift every score by log 2 and change nothing
   landmarks)      else; first/last-token landmark scores against numpy logaddexp and their
                   lexsort; central differences of dQ, dK, dV and dKlm; decode steps with
                   several landmarks equal prefill rows)
  decode_paged     pinned (equal to per-sequence contiguous decode steps over the gathered
                   pages, pages shuffled; with and without landmark-free chunks)
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hils_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DT_BF16 = 0
DT_F32 = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over independent rows / heads)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.oracle_landmark_scores.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, dbl, ip, ip]
    lib.oracle_landmark_scores.restype = None
    lib.oracle_landmark_scores_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, dbl, ip, vp, i64, ip]
    lib.oracle_landmark_scores_rows.restype = None
    lib.oracle_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, ip, vp, i64, ip, vp,
                               vp, vp, vp, vp, vp, ip]
    lib.oracle_fwd.restype = ip
    lib.oracle_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, dbl,
                                  ip, vp, vp, vp, vp, vp, ip, ip]
    lib.oracle_decode.restype = ip
    lib.oracle_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, ip, vp, vp,
                               vp, vp, vp, ip]
    lib.oracle_bwd.restype = ip
    lib.oracle_chunk_means.argtypes = [vp, i64, vp, i64, i64, i64, i64, i64, i64, ip, ip]
    lib.oracle_chunk_means.restype = None
    lib.oracle_fwd_lf.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, ip, vp, i64, ip,
                                  vp, vp, vp, vp, vp, ip]
    lib.oracle_fwd_lf.restype = ip
    lib.oracle_decode_lf.argtypes = lib.oracle_decode.argtypes
    lib.oracle_decode_lf.restype = ip
    lib.oracle_bwd_lf.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, ip, vp, vp, vp, vp,
                                  vp, ip]
    lib.oracle_bwd_lf.restype = ip
    lib.oracle_fwd_ml.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, dbl, ip, vp, i64, ip,
                                  vp, vp, vp, vp, vp, ip]
    lib.oracle_fwd_ml.restype = ip
    lib.oracle_decode_ml.argtypes = lib.oracle_decode.argtypes[:7] + [i64] + lib.oracle_decode.argtypes[7:]
    lib.oracle_decode_ml.restype = ip
    lib.oracle_bwd_ml.argtypes = [vp, vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64, i64, i64, dbl, ip, vp, vp,
                                  vp, vp, vp, ip]
    lib.oracle_bwd_ml.restype = ip
    _lib = lib
    return lib


def _dt(*arrs):
    kinds = {a.dtype for a in arrs}
    if len(kinds) != 1:
        raise TypeError(f"mixed input dtypes {kinds}")
    k = kinds.pop()
    if k == np.uint16:
        return DT_BF16
    if k == np.float32:
        return DT_F32
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {k}")


def _c(a):
    return np.ascontiguousarray(a)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def landmark_scores(Q, Klm, C, scale=None, nthreads=0):
    """S[b,h,t,j] = fp32(scale*<q_t, Klm_j>) for j <= t//C, -inf above; returned as float64."""
    Q, Klm = _c(Q), _c(Klm)
    B, H, L, d = Q.shape
    N = Klm.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    S = np.empty((B, H, L, N), np.float64)
    _load().oracle_landmark_scores(_p(Q), _p(Klm), _p(S), B, H, L, d, C, scale, _dt(Q, Klm), nthreads)
    return S


def landmark_scores_rows(Q, Klm, C, rows, scale=None, nthreads=0):
    """Scores of the listed flattened rows ((b*H+h)*L+t): [len(rows), N] float64."""
    Q, Klm = _c(Q), _c(Klm)
    B, H, L, d = Q.shape
    N = Klm.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    rows = _c(np.asarray(rows, np.int64))
    S = np.empty((rows.shape[0], N), np.float64)
    _load().oracle_landmark_scores_rows(_p(Q), _p(Klm), _p(S), B, H, L, d, C, scale, _dt(Q, Klm), _p(rows),
                                        rows.shape[0], nthreads)
    return S


def fwd(Q, K, V, Klm, C, k, scale=None, rows=None, idx=None, override_scores=None, nthreads=0, Q_ret=None):
    """Forward of every row (or of the flattened rows listed in ``rows``).

    Returns a dict with idx [.., k+1] int32, sel / w / lse [.., k+1] float64,
    O [.., d] float64 and ``threads`` (threads used).  With ``rows`` the leading
    shape is [len(rows)].  ``idx`` (same shape as the output idx) fixes the
    selection; ``override_scores`` [B,H,L,N] float64 replaces the landmark
    scores for selection and fusion.  ``Q_ret`` (same shape and type as Q):
    retrieval queries used for the landmark scores instead of Q.
    """
    Q, K, V, Klm = _c(Q), _c(K), _c(V), _c(Klm)
    Qr = _c(Q_ret) if Q_ret is not None else None
    if Qr is not None and (Qr.shape != Q.shape or Qr.dtype != Q.dtype):
        raise ValueError("Q_ret must match Q in shape and type")
    B, H, L, d = Q.shape
    N = Klm.shape[2]
    if N != (L + C - 1) // C:
        raise ValueError("Klm must hold one row per chunk")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    k1 = k + 1
    if rows is not None:
        rows = _c(np.asarray(rows, np.int64))
        lead = (rows.shape[0],)
    else:
        lead = (B, H, L)
    use_idx = idx is not None
    idx_out = _c(np.array(idx, np.int32, copy=True)).reshape(lead + (k1,)) if use_idx else np.empty(lead + (k1,), np.int32)
    sel = np.empty(lead + (k1,), np.float64)
    w = np.empty(lead + (k1,), np.float64)
    lse = np.empty(lead + (k1,), np.float64)
    O = np.empty(lead + (d,), np.float64)
    ov = _c(np.asarray(override_scores, np.float64)) if override_scores is not None else None
    used = _load().oracle_fwd(_p(Q), _p(Qr), _p(K), _p(V), _p(Klm), B, H, L, d, C, k, scale, _dt(Q, K, V, Klm),
                              _p(rows), 0 if rows is None else rows.shape[0], int(use_idx), _p(ov),
                              _p(idx_out), _p(sel), _p(w), _p(lse), _p(O), nthreads)
    return {"idx": idx_out, "sel": sel, "w": w, "lse": lse, "O": O, "threads": used}


def chunk_means(K, C, nchunks=None, Klm=None, nthreads=0):
    """Landmark-free chunk keys: row j = mean of key rows jC..jC+C-1 of every (b,h), rounded to fp32 and
    then to K's element type.  Fills ``Klm`` ([B,H,Nlm,d], K's type) in place for the first ``nchunks``
    chunks (default: every complete chunk) or returns a new [B,H,L//C,d] array."""
    K = _c(K)
    B, H, Lk, d = K.shape
    nchunks = Lk // C if nchunks is None else nchunks
    if nchunks * C > Lk:
        raise ValueError("nchunks exceeds the complete chunks of K")
    if Klm is None:
        Klm = np.zeros((B, H, Lk // C, d), K.dtype)
    if not Klm.flags.c_contiguous or Klm.dtype != K.dtype or Klm.shape[2] < nchunks:
        raise ValueError("Klm must be a C-contiguous array of K's type with room for the chunks")
    _load().oracle_chunk_means(_p(K), Lk, _p(Klm), Klm.shape[2], B, H, nchunks, d, C, _dt(K), nthreads)
    return Klm


def fwd_lf(Q, K, V, C, k, scale=None, rows=None, idx=None, nthreads=0, Q_ret=None):
    """Forward with landmark-free chunks: past chunks are scored by their key means, the own chunk by the
    mean of its keys up to the query.  Returns what ``fwd`` returns plus ``Klm`` (the key means)."""
    Q, K, V = _c(Q), _c(K), _c(V)
    Qr = _c(Q_ret) if Q_ret is not None else None
    if Qr is not None and (Qr.shape != Q.shape or Qr.dtype != Q.dtype):
        raise ValueError("Q_ret must match Q in shape and type")
    B, H, L, d = Q.shape
    if L % C:
        raise ValueError("L must be a multiple of C")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    k1 = k + 1
    if rows is not None:
        rows = _c(np.asarray(rows, np.int64))
        lead = (rows.shape[0],)
    else:
        lead = (B, H, L)
    use_idx = idx is not None
    idx_out = _c(np.array(idx, np.int32, copy=True)).reshape(lead + (k1,)) if use_idx else np.empty(lead + (k1,), np.int32)
    sel = np.empty(lead + (k1,), np.float64)
    w = np.empty(lead + (k1,), np.float64)
    lse = np.empty(lead + (k1,), np.float64)
    O = np.empty(lead + (d,), np.float64)
    Klm = np.zeros((B, H, L // C, d), K.dtype)
    used = _load().oracle_fwd_lf(_p(Q), _p(Qr), _p(K), _p(V), _p(Klm), B, H, L, d, C, k, scale, _dt(Q, K, V),
                                 _p(rows), 0 if rows is None else rows.shape[0], int(use_idx),
                                 _p(idx_out), _p(sel), _p(w), _p(lse), _p(O), nthreads)
    if used < 0:
        raise ValueError("unsupported shape")
    return {"idx": idx_out, "sel": sel, "w": w, "lse": lse, "O": O, "Klm": Klm, "threads": used}


def decode(q, k_new, v_new, Kc, Vc, Klm, n, C, k, scale=None, nthreads=0, q_ret=None, landmark_free=False,
           idx=None):
    """One decode step at position n for every (b,h).

    Writes k_new / v_new into row n of ``Kc`` / ``Vc`` in place (these are the
    caller's host arrays, [B,H,Lmax,d]) and returns idx / sel / w / lse [B,H,k+1]
    and o [B,H,d].  ``q_ret`` (like q): retrieval queries for the landmark scores.
    ``landmark_free``: landmark row n//C of ``Klm`` (updated in place) becomes the mean of the open
    chunk's keys so far; earlier rows are read as given (the key means of their chunks).
    ``idx`` [B,H,k+1] (optional): the selection held fixed; the step scores, weights and attends to
    these chunks (slots with -1 unused) instead of selecting its own, as ``fwd`` does with ``idx``.
    """
    q, k_new, v_new = _c(q), _c(k_new), _c(v_new)
    if landmark_free and not Klm.flags.c_contiguous:
        raise ValueError("Klm must be C-contiguous (it is updated in place)")
    Klm = Klm if landmark_free else _c(Klm)
    qr = _c(q_ret) if q_ret is not None else None
    if qr is not None and (qr.shape != q.shape or qr.dtype != q.dtype):
        raise ValueError("q_ret must match q in shape and type")
    if not (Kc.flags.c_contiguous and Vc.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous (they are updated in place)")
    B, H, d = q.shape
    Lmax = Kc.shape[2]
    Nmax = Klm.shape[2]
    if not (0 <= n < Lmax) or n // C >= Nmax:
        raise ValueError("n out of range")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    k1 = k + 1
    use_idx = idx is not None
    idx = _c(np.array(idx, np.int32, copy=True)).reshape(B, H, k1) if use_idx else np.empty((B, H, k1), np.int32)
    sel = np.empty((B, H, k1), np.float64)
    w = np.empty((B, H, k1), np.float64)
    lse = np.empty((B, H, k1), np.float64)
    o = np.empty((B, H, d), np.float64)
    tail = (n, Lmax, Nmax, B, H, d, C, k, scale, _dt(q, k_new, v_new, Kc, Vc, Klm), _p(idx), _p(sel), _p(w), _p(lse),
            _p(o), nthreads, int(use_idx))
    head = (_p(q), _p(qr), _p(k_new), _p(v_new), _p(Kc), _p(Vc), _p(Klm))
    if Klm.ndim == 5:
        # several landmarks per chunk: Klm [B,H,Nmax,m,d]
        if landmark_free:
            raise ValueError("landmark-free decode takes one landmark per chunk")
        used = _load().oracle_decode_ml(*head, Klm.shape[3], *tail)
    else:
        fn = _load().oracle_decode_lf if landmark_free else _load().oracle_decode
        used = fn(*head, *tail)
    if used < 0:
        raise ValueError("unsupported shape")
    return {"idx": idx, "sel": sel, "w": w, "lse": lse, "o": o, "threads": used}


def bwd(Q, K, V, Klm, dO, idx, C, k, scale=None, nthreads=0, Q_ret=None):
    """Gradients dQ, dK, dV [B,H,L,d] and dKlm [B,H,N,d] (float64), selection fixed by idx.

    With ``Q_ret`` (retrieval queries for the landmark scores) the score gradients go to a
    separate ``dQ_ret`` [B,H,L,d] and dQ holds the in-chunk attention terms only.
    """
    Q, K, V, Klm, dO = _c(Q), _c(K), _c(V), _c(Klm), _c(dO)
    Qr = _c(Q_ret) if Q_ret is not None else None
    if Qr is not None and (Qr.shape != Q.shape or Qr.dtype != Q.dtype):
        raise ValueError("Q_ret must match Q in shape and type")
    B, H, L, d = Q.shape
    N = Klm.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    idx = _c(np.asarray(idx, np.int32))
    if idx.shape != (B, H, L, k + 1):
        raise ValueError("idx must be [B,H,L,k+1]")
    dQ = np.empty((B, H, L, d), np.float64)
    dK = np.empty((B, H, L, d), np.float64)
    dV = np.empty((B, H, L, d), np.float64)
    dKlm = np.empty((B, H, N, d), np.float64)
    dQr = np.empty((B, H, L, d), np.float64) if Qr is not None else None
    used = _load().oracle_bwd(_p(Q), _p(Qr), _p(K), _p(V), _p(Klm), _p(dO), _p(idx), B, H, L, d, C, k, scale,
                              _dt(Q, K, V, Klm, dO), _p(dQ), _p(dQr), _p(dK), _p(dV), _p(dKlm), nthreads)
    out = {"dQ": dQ, "dK": dK, "dV": dV, "dKlm": dKlm, "threads": used}
    if Qr is not None:
        out["dQ_ret"] = dQr
    return out


def bwd_lf(Q, K, V, dO, idx, C, k, scale=None, nthreads=0, Q_ret=None):
    """Backward of ``fwd_lf`` with the selection fixed by idx: dQ, dK, dV [B,H,L,d] (float64), dK including the
    landmark paths (the key means), and dKlm [B,H,N,d], the gradient with respect to the past chunks' means.
    With ``Q_ret`` the score gradients go to ``dQ_ret``."""
    Q, K, V, dO = _c(Q), _c(K), _c(V), _c(dO)
    Qr = _c(Q_ret) if Q_ret is not None else None
    if Qr is not None and (Qr.shape != Q.shape or Qr.dtype != Q.dtype):
        raise ValueError("Q_ret must match Q in shape and type")
    B, H, L, d = Q.shape
    if L % C:
        raise ValueError("L must be a multiple of C")
    N = L // C
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    idx = _c(np.asarray(idx, np.int32))
    dQ, dK, dV = (np.empty((B, H, L, d), np.float64) for _ in range(3))
    dKlm = np.empty((B, H, N, d), np.float64)
    dQr = np.empty((B, H, L, d), np.float64) if Qr is not None else None
    used = _load().oracle_bwd_lf(_p(Q), _p(Qr), _p(K), _p(V), _p(dO), _p(idx), B, H, L, d, C, k, scale,
                                 _dt(Q, K, V, dO), _p(dQ), _p(dQr), _p(dK), _p(dV), _p(dKlm), nthreads)
    if used < 0:
        raise ValueError("unsupported shape")
    out = {"dQ": dQ, "dK": dK, "dV": dV, "dKlm": dKlm, "threads": used}
    if Qr is not None:
        out["dQ_ret"] = dQr
    return out


def decode_paged(q, k_new, v_new, Kp, Vp, Klm_p, page_table, n_ctx, C, k, scale=None, nthreads=0, q_ret=None,
                 landmark_free=False, idx=None):
    """One decode step of B sequences at positions n_ctx[b] over page pools Kp, Vp [P,H,C,d], Klm_p [P,H,d]
    (or [P,H,m,d]: m landmarks per chunk) (host arrays, updated in place) with page_table [B,max_pages].
    Paging only moves rows: each sequence's chunks 0..n_ctx[b]//C are gathered into contiguous caches,
    ``decode`` runs there, and the rows it writes go back to their pages.  ``idx`` [B,H,k+1] (optional):
    the selection held fixed.  Returns idx / sel / w / lse [B,H,k+1] and o [B,H,d]."""
    B, H, d = q.shape
    maxp = page_table.shape[1]
    Lmax = maxp * C
    outs = []
    for b in range(B):
        n = int(n_ctx[b])
        c = n // C
        pages = [int(page_table[b, j]) for j in range(c + 1)]
        Kc = np.zeros((1, H, Lmax, d), Kp.dtype)
        Vc = np.zeros_like(Kc)
        Klm = np.zeros((1, H, maxp) + Klm_p.shape[2:], Klm_p.dtype)
        for j, p in enumerate(pages):
            Kc[0, :, j * C:(j + 1) * C] = Kp[p]
            Vc[0, :, j * C:(j + 1) * C] = Vp[p]
            Klm[0, :, j] = Klm_p[p]
        r = decode(q[b:b + 1], k_new[b:b + 1], v_new[b:b + 1], Kc, Vc, Klm, n, C, k, scale=scale, nthreads=nthreads,
                   q_ret=None if q_ret is None else q_ret[b:b + 1], landmark_free=landmark_free,
                   idx=None if idx is None else idx[b:b + 1])
        Kp[pages[c], :, n - c * C] = Kc[0, :, n]
        Vp[pages[c], :, n - c * C] = Vc[0, :, n]
        if landmark_free:
            Klm_p[pages[c]] = Klm[0, :, c]
        outs.append(r)
    return {key: np.concatenate([r[key] for r in outs]) for key in ("idx", "sel", "w", "lse", "o")}


def fwd_ml(Q, K, V, Klm, C, k, scale=None, rows=None, idx=None, nthreads=0, Q_ret=None):
    """Forward with m landmarks per chunk (Klm [B,H,N,m,d]): the chunk score is the log-sum-exp of the
    chunk's landmark scores.  Returns what ``fwd`` returns."""
    Q, K, V, Klm = _c(Q), _c(K), _c(V), _c(Klm)
    Qr = _c(Q_ret) if Q_ret is not None else None
    B, H, L, d = Q.shape
    N, m = Klm.shape[2], Klm.shape[3]
    if N != (L + C - 1) // C or Klm.shape[4] != d:
        raise ValueError("Klm must be [B,H,N,m,d]")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    k1 = k + 1
    if rows is not None:
        rows = _c(np.asarray(rows, np.int64))
        lead = (rows.shape[0],)
    else:
        lead = (B, H, L)
    use_idx = idx is not None
    idx_out = _c(np.array(idx, np.int32, copy=True)).reshape(lead + (k1,)) if use_idx else np.empty(lead + (k1,), np.int32)
    sel, w, lse = (np.empty(lead + (k1,), np.float64) for _ in range(3))
    O = np.empty(lead + (d,), np.float64)
    used = _load().oracle_fwd_ml(_p(Q), _p(Qr), _p(K), _p(V), _p(Klm), m, B, H, L, d, C, k, scale, _dt(Q, K, V, Klm),
                                 _p(rows), 0 if rows is None else rows.shape[0], int(use_idx),
                                 _p(idx_out), _p(sel), _p(w), _p(lse), _p(O), nthreads)
    if used < 0:
        raise ValueError("unsupported landmark count")
    return {"idx": idx_out, "sel": sel, "w": w, "lse": lse, "O": O, "threads": used}


def bwd_ml(Q, K, V, Klm, dO, idx, C, k, scale=None, nthreads=0, Q_ret=None):
    """Backward of ``fwd_ml`` with the selection fixed by idx: dQ, dK, dV [B,H,L,d], dKlm [B,H,N,m,d] (float64),
    and dQ_ret with ``Q_ret``."""
    Q, K, V, Klm, dO = _c(Q), _c(K), _c(V), _c(Klm), _c(dO)
    Qr = _c(Q_ret) if Q_ret is not None else None
    B, H, L, d = Q.shape
    N, m = Klm.shape[2], Klm.shape[3]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    idx = _c(np.asarray(idx, np.int32))
    dQ, dK, dV = (np.empty((B, H, L, d), np.float64) for _ in range(3))
    dKlm = np.empty((B, H, N, m, d), np.float64)
    dQr = np.empty((B, H, L, d), np.float64) if Qr is not None else None
    used = _load().oracle_bwd_ml(_p(Q), _p(Qr), _p(K), _p(V), _p(Klm), m, _p(dO), _p(idx), B, H, L, d, C, k, scale,
                                 _dt(Q, K, V, Klm, dO), _p(dQ), _p(dQr), _p(dK), _p(dV), _p(dKlm), nthreads)
    if used < 0:
        raise ValueError("unsupported landmark count")
    out = {"dQ": dQ, "dK": dK, "dV": dV, "dKlm": dKlm, "threads": used}
    if Qr is not None:
        out["dQ_ret"] = dQr
    return out
