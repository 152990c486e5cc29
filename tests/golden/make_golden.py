"""Writes the worked examples under tests/golden/ from their closed forms (numpy only: no oracle, no
GPU library).  Run from the repository root: python tests/golden/make_golden.py

fusion_ties_6chunks.json -- the operator of "Hierarchical Sparse Attention Done Right" (ai-feeds
summary, "Method" > "Key modules" items 1-3: landmark scores, causal top-k of the past chunks, attention
inside each kept chunk, fusion by a softmax over the kept chunks' scores), with the readings fixed for
this library: one landmark per chunk, scale 1/sqrt(d), ties toward the lower chunk index, the own chunk
always kept and scored by its landmark.

Construction (C = 64, six chunks, d = 64, k = 2): every query row is e_0; landmark j is alpha_j e_0, so
the score of chunk j is alpha_j / 8 for every query; every key is 0, so attention inside a chunk is
uniform; every value row of chunk j is v_j = (j + 1) e_0 - (j + 1) / 2 e_1, so a chunk's output is v_j
whatever the query's position inside the chunk (the own chunk's causal prefix included).  A query in
chunk c therefore keeps the two past chunks of largest alpha (lower index first on ties) plus chunk c,
and its output is sum_j w_j v_j with w the softmax of the kept scores.  alpha has a tie (chunks 1 and
2) that decides the selection of chunk 3's queries.  The gradients for dO = e_0 follow the same way
(see backward()); the backward's passages are the chatpaper abstract (the retrieval scores are trained
through the fused output) and the ai-feeds summary's "Output & training".
"""
import json
import math
import os

C, N, D, K = 64, 6, 64, 2
SCALE = 1.0 / math.sqrt(D)
ALPHA = [3.0, 2.0, 2.0, 5.0, 1.0, 4.0]


def v(j):
    return (j + 1.0, -(j + 1.0) / 2.0)


def chunk_case(c):
    past = sorted(range(c), key=lambda j: (-ALPHA[j], j))[:K]
    kept = past + [c]
    s = [SCALE * ALPHA[j] for j in kept]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    tot = sum(e)
    wk = [x / tot for x in e]
    idx = past + [-1] * (K - len(past)) + [c]
    sel = s[:len(past)] + [None] * (K - len(past)) + [s[-1]]
    w = wk[:len(past)] + [0.0] * (K - len(past)) + [wk[-1]]
    o = [sum(wj * v(j)[i] for wj, j in zip(wk, kept)) for i in range(2)]
    return {"c": c, "idx": idx, "sel": sel, "w": w, "o01": o}


def backward():
    """Gradients for the upstream gradient dO = e_0 on every row, from the chain rule by hand.  Inside a
    kept chunk every value row is v_j, so D_j = dO . o_j = j + 1 and the in-chunk score gradients
    w_j p_i (dO . v_i - D_j) vanish: dK = 0 and dQ has only the fusion term.  With D = sum_j w_j D_j
    and ds_j = w_j (D_j - D): dQ_t = scale sum_j ds_j alpha_j e_0, dK_lm[j] = scale sum_t ds_tj e_0,
    and dV_i = sum_t w_tj p_ti e_0, where p_ti = 1/64 over a past chunk and 1/(t - 64 c + 1) over the
    own chunk's causal prefix."""
    L = C * N
    dq0 = [0.0] * L
    dv0 = [0.0] * L
    dklm0 = [0.0] * N
    for t in range(L):
        c = t // C
        case = chunk_case(c)
        kept = [j for j in case["idx"] if j >= 0]
        wk = [case["w"][s] for s, j in enumerate(case["idx"]) if j >= 0]
        dj = [j + 1.0 for j in kept]
        dd = sum(w * x for w, x in zip(wk, dj))
        ds = [w * (x - dd) for w, x in zip(wk, dj)]
        dq0[t] = SCALE * sum(g * ALPHA[j] for g, j in zip(ds, kept))
        for g, j, w in zip(ds, kept, wk):
            dklm0[j] += SCALE * g
            keys = range(j * C, (j + 1) * C) if j < c else range(c * C, t + 1)
            for i in keys:
                dv0[i] += w / len(keys)
    return {"dO": "e_0 on every row", "dQ0": dq0, "dV0": dv0, "dKlm0": dklm0}


def main():
    out = {
        "source": "Hierarchical Sparse Attention Done Right (ai-feeds summary), Method > Key modules items 1-3",
        "construction": "q = e_0 on every row; K_lm[j] = alpha_j e_0; K = 0; V rows of chunk j = (j+1) e_0 - (j+1)/2 e_1",
        "C": C, "N": N, "d": D, "k": K, "scale": SCALE, "alpha": ALPHA,
        "per_query_chunk": [chunk_case(c) for c in range(N)],
        "backward": backward(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fusion_ties_6chunks.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
