"""Parity of the batched decode step over a paged cache with the CPU oracle.

Serving shapes: B sequences at ragged positions, each chunk of 64 tokens in its own pool page,
pages in a shuffled order; optionally with retrieval queries and landmark-free chunks.
"""
import numpy as np
import pytest
import torch

import oracle
from long_context_landmark_amd import synth
from gpu_util import assert_close, check_decode_step, dev, f32, host, say, tol

pytestmark = pytest.mark.gpu


def _build(B, H, d, ctxs, steps, dtype, lf, rq, seed, m=1):
    C = 64
    rng = np.random.default_rng(seed)
    xs = [synth.decode_inputs(1, H, d, ctx, steps, C=C, seed=seed + b, dtype=dtype, with_qret=rq)
          for b, ctx in enumerate(ctxs)]
    nchunks = [(ctx + steps - 1) // C + 1 for ctx in ctxs]
    maxp = max(nchunks) + 2
    total = sum(nchunks) + 5
    order = rng.permutation(total)
    table = np.zeros((B, maxp), np.int32)
    etype = xs[0]["K_cache"].dtype
    Kp = np.zeros((total, H, C, d), etype)
    Vp = np.zeros_like(Kp)
    Lp = np.zeros((total, H) + ((m, d) if m > 1 else (d,)), etype)
    nxt = 0
    for b, x in enumerate(xs):
        Klm_b = x["Klm"].copy()
        if m > 1:
            # several landmarks per chunk: the given row and m - 1 further N(0,1) rows
            extra = rng.standard_normal(Klm_b.shape[:3] + (m - 1, d), dtype=np.float32)
            extra = synth.f32_to_bf16_bits(extra) if dtype == "bf16" else extra
            Klm_b = np.concatenate([Klm_b[:, :, :, None], extra], axis=3)
        if lf:
            Klm_b[:] = 0
            oracle.chunk_means(x["K_cache"], C, nchunks=ctxs[b] // C, Klm=Klm_b)
        for j in range(nchunks[b]):
            p = int(order[nxt])
            nxt += 1
            table[b, j] = p
            rows = x["K_cache"][0, :, j * C:(j + 1) * C]
            Kp[p, :, :rows.shape[1]] = rows
            Vp[p, :, :rows.shape[1]] = x["V_cache"][0, :, j * C:(j + 1) * C]
            if j < Klm_b.shape[2]:
                Lp[p] = Klm_b[0, :, j]
    return xs, Kp, Vp, Lp, table


@pytest.mark.parametrize("dtype,H,d,ctxs,steps,k,lf,rq,m", [
    ("bf16", 2, 64, [64 * 40 + 10, 64 * 7 + 60, 3], 70, 4, False, False, 1),
    ("bf16", 2, 128, [64 * 300 + 62, 64 * 2, 64 * 17 + 33], 4, 16, False, True, 1),
    ("bf16", 2, 64, [64 * 25 + 50, 64 * 9 + 1], 30, 8, True, True, 1),
    ("f32", 1, 64, [64 * 20, 64 * 3 + 63], 20, 4, True, False, 1),
    # several landmarks per page: log-sum-exp chunk scores
    ("bf16", 2, 64, [64 * 40 + 10, 64 * 7 + 60, 3], 70, 4, False, False, 2),
    ("bf16", 2, 128, [64 * 300 + 62, 64 * 17 + 33], 4, 16, False, True, 3),
    ("f32", 1, 64, [64 * 20, 64 * 3 + 63], 20, 4, False, False, 2),
])
def test_decode_paged(hils, gpu, dtype, H, d, ctxs, steps, k, lf, rq, m):
    B = len(ctxs)
    say(f"paged decode dtype={dtype} B={B} H={H} d={d} ctx={ctxs} steps={steps} k={k} lf={lf} retrieval={rq} m={m}")
    xs, Kp, Vp, Lp, table = _build(B, H, d, ctxs, steps, dtype, lf, rq, seed=700 + d + steps + m, m=m)
    Kp_g, Vp_g, Lp_g = dev(Kp), dev(Vp), dev(Lp)
    table_g = torch.from_numpy(table).to(gpu)
    maxp = table.shape[1]
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, maxp * 64, d, 64, k), dtype=torch.uint8, device=gpu)
    bar = tol(dtype)
    near = 0
    for s in range(steps):
        pos = np.array([ctx + s for ctx in ctxs], np.int64)
        q = np.stack([x["q"][s][0] for x in xs])
        kn = np.stack([x["k_new"][s][0] for x in xs])
        vn = np.stack([x["v_new"][s][0] for x in xs])
        qr = np.stack([x["q_ret"][s][0] for x in xs]) if rq else None
        o, idx, w = hils.decode_step_paged(dev(q), dev(kn), dev(vn), Kp_g, Vp_g, Lp_g, table_g,
                                           torch.from_numpy(pos).to(gpu), int(pos.max()), k,
                                           q_ret=dev(qr) if rq else None, landmark_free=lf, ws=ws)
        step = lambda sel=None: oracle.decode_paged(q, kn, vn, Kp, Vp, Lp, table, pos, 64, k, q_ret=qr,
                                                    landmark_free=lf,
                                                    idx=None if sel is None else sel.reshape(B, H, k + 1))
        ref = step()
        torch.cuda.synchronize()
        own = [int(pos[bh // H]) // 64 for bh in range(B * H)]

        def past(bh, q=q, qr=qr, own=own):
            b, h = divmod(bh, H)
            c = own[bh]
            qf = synth.as_f32((qr if rq else q)[b, h]).astype(np.float64)
            lm = synth.as_f32(np.stack([Lp[table[b, j], h] for j in range(c)])).astype(np.float64)
            sc = lm @ qf / np.sqrt(d)
            if m > 1:  # log-sum-exp over the chunk's landmarks
                sc = np.log(np.exp(sc - sc.max(1, keepdims=True)).sum(1)) + sc.max(1)
            return sc.astype(np.float32)

        near += check_decode_step(f"step {s}", idx.cpu().numpy().reshape(B * H, k + 1),
                                  f32(w).reshape(B * H, k + 1), f32(o).reshape(B * H, d), ref, step, own, past, k,
                                  bar)
    say(f"  rows with near-tie selection differences: {near}")
    np.testing.assert_array_equal(host(Kp_g), Kp)
    np.testing.assert_array_equal(host(Vp_g), Vp)
    if lf:
        g, r = synth.as_f32(host(Lp_g)).astype(np.float64), synth.as_f32(Lp).astype(np.float64)
        np.testing.assert_allclose(g, r, rtol=2.0 ** -7 if dtype == "bf16" else 1e-5, atol=1e-6)
    else:
        np.testing.assert_array_equal(host(Lp_g), Lp)
