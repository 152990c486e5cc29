"""The entry points can be captured in a HIP graph and replayed: every replay equals the eager result.

The library launches only kernels on the caller's stream (no allocation, no memset, no host sync), which is
what the benchmark relies on when it replays a captured step.
"""
import numpy as np
import pytest
import torch

from long_context_landmark_amd import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def test_fwd_graph_replays_match_eager(hils, gpu):
    B, H, L, d, k = 1, 4, 4096, 64, 8
    say(f"graph fwd B={B} H={H} L={L} d={d} k={k}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=9, dtype="bf16", klm="chunkmean")
    Q, K, V, Klm = (dev(x[n]) for n in ("Q", "K", "V", "Klm"))
    ws = torch.empty(hils.workspace_size(hils.OP_FWD, B, H, L, d, 64, k), dtype=torch.uint8, device=gpu)
    O = torch.empty_like(Q)
    ref = [t.clone() for t in hils.sparse_attn_fwd(Q, K, V, Klm, k, ws=ws, save_for_backward=True)]
    torch.cuda.synchronize()
    out = {}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out["r"] = hils.sparse_attn_fwd(Q, K, V, Klm, k, ws=ws, out=O, save_for_backward=True)
    for rep in range(4):
        # unrelated eager work on the same buffers between replays
        hils.sparse_attn_fwd(K, Q, V, Klm, k, ws=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out["r"], ref):
            assert torch.equal(a, b), f"replay {rep} differs"


def test_decode_graph_replays_match_eager(hils, gpu):
    B, H, d, k = 1, 4, 64, 8
    ctx, steps = 64 * 200 + 30, 40
    say(f"graph decode B={B} H={H} d={d} ctx={ctx} steps={steps} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=12, dtype="bf16")
    Lmax = ctx + steps
    Kc0, Vc0, Klm = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
    q, kn, vn = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, k), dtype=torch.uint8, device=gpu)
    Kc, Vc = Kc0.clone(), Vc0.clone()
    ref = []
    for s in range(steps):
        o, i, w = hils.decode_step(q[s], kn[s], vn[s], Kc, Vc, Klm, ctx + s, k, ws=ws)
        ref.append((o.clone(), i.clone(), w.clone()))
    torch.cuda.synchronize()
    Kc2, Vc2 = Kc0.clone(), Vc0.clone()
    outs = [(torch.empty_like(r[0]), torch.empty_like(r[1]), torch.empty_like(r[2])) for r in ref]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(steps):
            hils.decode_step(q[s], kn[s], vn[s], Kc2, Vc2, Klm, ctx + s, k, ws=ws, out=outs[s][0], idx=outs[s][1],
                             w=outs[s][2])
    for rep in range(3):
        hils.decode_step(q[0], kn[0], vn[0], Kc.clone(), Vc.clone(), Klm, ctx, k, ws=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            for a, b in zip(outs[s], ref[s]):
                assert torch.equal(a, b), f"replay {rep} step {s} differs"
        assert torch.equal(Kc2, Kc) and torch.equal(Vc2, Vc)
