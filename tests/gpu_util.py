"""Helpers of the GPU parity tests: device transfer, the selection gap rule, error norms."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from long_context_landmark_amd import synth

# parity bar for bf16 inputs (floating outputs) and for selections
MAX_ABS = 2e-2
REL_L2 = 1e-2
GAP = 1e-4
# fp32 inputs: every intermediate stays fp32 (MFMA fp32 products, fp32 per-pair rows, fp32 sums), so the
# outputs are held to single-precision rounding of the double-precision oracle: a few hundred fp32 ulps of
# unit-scale values at most, and a relative L2 error of a few ulps
F32_MAX_ABS = 1e-4
F32_REL_L2 = 1e-5


def tol(dtype):
    """(max-abs, rel-L2) bar of an input type."""
    return (F32_MAX_ABS, F32_REL_L2) if dtype == "f32" else (MAX_ABS, REL_L2)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    """Host array (uint16 bf16 bits or float32) -> contiguous tensor on cuda:0."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x.copy()).to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array in the oracle's input representation."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def errs(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)) if d.size else 0.0
    return max_abs, rel


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = errs(got, ref)
    say(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"


def selection_sets(idx: np.ndarray, k: int):
    """Past-chunk sets of each row of an idx array [..., k+1] (flattened rows)."""
    flat = idx.reshape(-1, k + 1)
    return [frozenset(int(j) for j in row[:k] if j >= 0) for row in flat]


def check_selection(gpu_idx, ora_idx, Q, Klm, C, k, rows=None):
    """Index sets must agree row by row; a differing chunk is allowed only when its oracle score lies within
    GAP of the oracle's m-th best score.  Returns the flattened row numbers (into ``rows`` if given) whose sets
    differ."""
    g = gpu_idx.reshape(-1, k + 1)
    o = ora_idx.reshape(-1, k + 1)
    L = Q.shape[2]
    row_ids = np.arange(g.shape[0]) if rows is None else np.asarray(rows)
    t_of = row_ids % L
    # own chunk and -1 padding are exact
    np.testing.assert_array_equal(g[:, k], t_of // C)
    np.testing.assert_array_equal(g[:, k], o[:, k])
    m_of = np.minimum(k, t_of // C)
    for r in range(g.shape[0]):
        assert np.all(g[r, m_of[r]:k] == -1), f"row {row_ids[r]}: padding {g[r]}"
    gs, os_ = selection_sets(g, k), selection_sets(o, k)
    bad = [r for r in range(len(gs)) if gs[r] != os_[r]]
    if bad:
        S = oracle.landmark_scores_rows(Q, Klm, C, row_ids[bad])
        worst = 0.0
        for i, r in enumerate(bad):
            m = int(m_of[r])
            assert len(gs[r]) == m, f"row {row_ids[r]}: {len(gs[r])} chunks kept, {m} expected"
            mth = np.sort(S[i, :t_of[r] // C].astype(np.float32))[::-1][m - 1]
            for j in gs[r] ^ os_[r]:
                gap = abs(float(S[i, j]) - float(mth))
                worst = max(worst, gap)
                assert gap < GAP, f"row {row_ids[r]}: chunk {j} differs with score gap {gap:.3e}"
        say(f"  selection: {len(bad)} of {len(gs)} rows differ on near ties (max gap {worst:.2e})")
    else:
        say(f"  selection: all {len(gs)} rows identical")
    return np.asarray(bad, np.int64)


def to_inputs(x, names=("Q", "K", "V", "Klm")):
    return {n: dev(x[n]) for n in names}


def check_decode_step(tag, gi, gw, go, ref, rerun, own, past_scores, k, tol=(MAX_ABS, REL_L2), w_tol=2e-5):
    """One decode step of R rows (flattened (b, h)) against the oracle.

    gi [R, k+1], gw [R, k+1], go [R, d]: the GPU's selection, weights and output.  ``ref``: the oracle's free
    step (idx [.., k+1]).  ``own[r]``: the open chunk of row r.  ``past_scores(r)``: the oracle-precision fp32
    scores of row r's past chunks 0..own[r]-1.  Selection: the own slot and the -1 padding are exact, and the
    past-chunk sets are equal or differ only in chunks whose score lies within GAP of the m-th best.
    Outputs: o and w of every row against the oracle step with the GPU's selection held fixed
    (``rerun(gi)``), so rows that differ on a near tie are checked too.  Returns the number of such rows."""
    R = gi.shape[0]
    ri = np.asarray(ref["idx"]).reshape(R, k + 1)
    differ = 0
    for r in range(R):
        c = int(own[r])
        m = min(k, c)
        assert gi[r, k] == c and np.all(gi[r, m:k] == -1), (tag, r, gi[r])
        a, b = set(gi[r, :m].tolist()), set(ri[r, :m].tolist())
        assert len(a) == m, (tag, r, gi[r])
        if a != b:
            sc = np.asarray(past_scores(r), np.float32)
            mth = np.sort(sc)[::-1][m - 1]
            for j in a ^ b:
                gap = abs(float(sc[j]) - float(mth))
                assert gap < GAP, (tag, r, j, gap)
            differ += 1
    fixed = rerun(gi)
    assert_close(go, np.asarray(fixed["o"]).reshape(go.shape), f"o {tag}", *tol)
    fw = np.asarray(fixed["w"]).reshape(R, k + 1)
    np.testing.assert_array_equal(np.asarray(fixed["idx"]).reshape(R, k + 1), gi)
    werr = float(np.max(np.abs(gw - fw)))
    assert werr < w_tol, (tag, werr)
    return differ
