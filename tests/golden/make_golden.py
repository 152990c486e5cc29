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
2) that decides the selection of chunk 3's queries.
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


def main():
    out = {
        "source": "Hierarchical Sparse Attention Done Right (ai-feeds summary), Method > Key modules items 1-3",
        "construction": "q = e_0 on every row; K_lm[j] = alpha_j e_0; K = 0; V rows of chunk j = (j+1) e_0 - (j+1)/2 e_1",
        "C": C, "N": N, "d": D, "k": K, "scale": SCALE, "alpha": ALPHA,
        "per_query_chunk": [chunk_case(c) for c in range(N)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fusion_ties_6chunks.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
