"""The decode step that allocates nothing (library-held scratch) against the workspace decode step.

Called through the C ABI: two calls in a row on the same GPU, the second with a smaller batch and a
shorter context, must give the same selection, weights, outputs and cache appends as hils_decode_step
with a caller workspace (same kernels: bit for bit)."""
import ctypes

import numpy as np
import pytest
import torch

from long_context_landmark_amd import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _ws_step(hils, x, s, Kc, Vc, Klm, n, k, ws):
    return hils.decode_step(dev(x["q"][s]), dev(x["k_new"][s]), dev(x["v_new"][s]), Kc, Vc, Klm, n, k, ws=ws)


def _noalloc_step(hils, x, s, Kc, Vc, Klm, n, k):
    B, H, d = x["q"][s].shape
    q, kn, vn = dev(x["q"][s]), dev(x["k_new"][s]), dev(x["v_new"][s])
    o = torch.empty_like(q)
    idx = torch.empty((B, H, k + 1), dtype=torch.int32, device=q.device)
    w = torch.empty((B, H, k + 1), dtype=torch.float32, device=q.device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = hils._lib.hils_decode_step_noalloc(P(q), P(kn), P(vn), P(Kc), P(Vc), P(Klm), n, Kc.shape[2], P(o), P(idx),
                                            P(w), B, H, d, 64, k, 1.0 / np.sqrt(d), hils.BF16,
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, hils._lib.hils_last_error().decode()
    return o, idx, w


@pytest.mark.parametrize("calls", [[(2, 8, 64, 64 * 1500 + 30, 16), (1, 3, 64, 64 * 200 + 5, 8)],
                                   [(1, 4, 128, 64 * 700 + 63, 16), (1, 2, 128, 64 * 3 + 1, 4)]])
def test_noalloc_decode_matches_workspace_decode(hils, gpu, calls):
    for i, (B, H, d, ctx, k) in enumerate(calls):
        say(f"no-alloc decode call {i}: B={B} H={H} d={d} ctx={ctx} k={k}")
        x = synth.decode_inputs(B, H, d, ctx, 2, C=64, seed=900 + i + d, dtype="bf16")
        Kc_a, Vc_a, Klm = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
        Kc_b, Vc_b = Kc_a.clone(), Vc_a.clone()
        ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Kc_a.shape[2], d, 64, k), dtype=torch.uint8,
                         device=gpu)
        for s in range(2):
            ra = _ws_step(hils, x, s, Kc_a, Vc_a, Klm, ctx + s, k, ws)
            rb = _noalloc_step(hils, x, s, Kc_b, Vc_b, Klm, ctx + s, k)
            torch.cuda.synchronize()
            for a, b in zip(ra, rb):
                assert torch.equal(a, b)
        assert torch.equal(Kc_a, Kc_b) and torch.equal(Vc_a, Vc_b)


def test_noalloc_decode_rejects_batches_above_the_scratch(hils, gpu):
    P = ctypes.c_void_p(0x10000)
    st = hils._lib.hils_decode_step_noalloc(P, P, P, P, P, P, 100, 1024, P, P, P, 1, 700, 128, 64, 8, 0.125,
                                            hils.BF16, None)
    assert st == 2 and "scratch" in hils._lib.hils_last_error().decode()


def test_noalloc_decode_graph_replays(hils, gpu):
    """The caller it is for: steps captured in a HIP graph (no allocation inside the capture) and replayed, each
    replay equal to the workspace step run eagerly, with unrelated eager steps between replays."""
    B, H, d, k = 1, 4, 64, 8
    ctx, steps = 64 * 300 + 20, 12
    say(f"no-alloc decode in a graph: B={B} H={H} d={d} ctx={ctx} steps={steps} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=41, dtype="bf16")
    Kc0, Vc0, Klm = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Kc0.shape[2], d, 64, k), dtype=torch.uint8, device=gpu)
    Kc, Vc = Kc0.clone(), Vc0.clone()
    ref = [tuple(t.clone() for t in _ws_step(hils, x, s, Kc, Vc, Klm, ctx + s, k, ws)) for s in range(steps)]
    q, kn, vn = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    outs = [(torch.empty_like(r[0]), torch.empty_like(r[1]), torch.empty_like(r[2])) for r in ref]
    Kc2, Vc2 = Kc0.clone(), Vc0.clone()
    # the first call on the device looks up the scratch address: made before the capture
    hils.decode_step_noalloc(q[0], kn[0], vn[0], Kc0.clone(), Vc0.clone(), Klm, ctx, k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(steps):
            hils.decode_step_noalloc(q[s], kn[s], vn[s], Kc2, Vc2, Klm, ctx + s, k, out=outs[s][0], idx=outs[s][1],
                                     w=outs[s][2])
    for rep in range(3):
        # eager calls between replays leave their own contents in the shared scratch
        hils.decode_step_noalloc(q[1], kn[1], vn[1], Kc0.clone(), Vc0.clone(), Klm, ctx + 1, k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            for a, b in zip(outs[s], ref[s]):
                assert torch.equal(a, b), f"replay {rep} step {s} differs"
        assert torch.equal(Kc2, Kc) and torch.equal(Vc2, Vc)
