"""Inputs of the worked examples under tests/golden/ (numpy only; no arithmetic of the method).

Both the oracle's pins and the GPU tests build their inputs here from the fixture's construction; the
expected values come from the fixture itself (closed forms, see tests/golden/make_golden.py)."""
import json
import os

import numpy as np

from long_context_landmark_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cast(x, dtype):
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def fusion_ties_prefill(g, dtype):
    """q = e_0 on every row, K = 0, V rows of chunk j = (j+1) e_0 - (j+1)/2 e_1, K_lm[j] = alpha_j e_0;
    shapes [1, 1, L, d] and [1, 1, N, d]."""
    C, N, d = g["C"], g["N"], g["d"]
    L = C * N
    Q = np.zeros((1, 1, L, d), np.float32)
    Q[..., 0] = 1.0
    K = np.zeros_like(Q)
    V = np.zeros_like(Q)
    for j in range(N):
        V[0, 0, j * C:(j + 1) * C, 0] = j + 1.0
        V[0, 0, j * C:(j + 1) * C, 1] = -(j + 1.0) / 2.0
    Klm = np.zeros((1, 1, N, d), np.float32)
    Klm[0, 0, :, 0] = np.asarray(g["alpha"], np.float32)
    return {n: _cast(a, dtype) for n, a in (("Q", Q), ("K", K), ("V", V), ("Klm", Klm))}


def fusion_ties_decode(g, n, dtype):
    """The same construction as a decode step at position n: caches hold rows 0..n-1 (row n is appended
    from k_new, v_new), landmark rows of every chunk; q, k_new, v_new [1, 1, d]."""
    x = fusion_ties_prefill(g, "f32")
    Kc, Vc, Klm = x["K"].copy(), x["V"].copy(), x["Klm"].copy()
    k_new = Kc[:, :, n].copy()
    v_new = Vc[:, :, n].copy()
    Kc[:, :, n:] = 0.0
    Vc[:, :, n:] = 0.0
    q = x["Q"][:, :, n].copy()
    return {n_: _cast(a, dtype) for n_, a in (("q", q), ("k_new", k_new), ("v_new", v_new), ("Kc", Kc), ("Vc", Vc),
                                              ("Klm", Klm))}


def fusion_ties_dO(g, dtype):
    """Upstream gradient e_0 on every row, [1, 1, L, d]."""
    dO = np.zeros((1, 1, g["C"] * g["N"], g["d"]), np.float32)
    dO[..., 0] = 1.0
    return _cast(dO, dtype)


def fusion_ties_idx(g):
    """The worked example's selection, [1, 1, L, k+1] int32 (every row of a query chunk the same)."""
    return np.repeat(np.array([c["idx"] for c in g["per_query_chunk"]], np.int32), g["C"], axis=0)[None, None]
