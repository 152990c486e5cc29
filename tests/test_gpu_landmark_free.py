"""Parity of the landmark-free entry points with the CPU oracle.

Landmark-free chunks (the alternative the HiLS summary page mentions under "Method" >
"Input & chunking"): a chunk's landmark is the mean of its keys; the query's own chunk
averages only the keys up to the query.  Each side forms its own means from the same keys.
"""
import numpy as np
import pytest
import torch

import oracle
from long_context_landmark_amd import synth
from gpu_util import assert_close, check_decode_step, check_selection, dev, f32, host, say, to_inputs, tol
from test_gpu_decode import past_scores_fn

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return tol(dtype)


def _means_close(got, ref, dtype, what):
    """fp32 sums in another order: bf16 means agree except on rare rounding ties (one bf16 step apart)."""
    g, r = synth.as_f32(got).astype(np.float64), synth.as_f32(ref).astype(np.float64)
    if dtype == "bf16":
        exact = np.mean(g == r)
        say(f"  {what}: {exact * 100:.3f}% of elements bit-exact")
        assert exact > 0.999
        np.testing.assert_allclose(g, r, rtol=2.0 ** -7, atol=1e-30)
    else:
        np.testing.assert_allclose(g, r, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_chunk_means(hils, gpu, dtype, d):
    say(f"chunk means dtype={dtype} d={d}")
    x = synth.prefill_inputs(2, 3, 64 * 21, d, C=64, seed=600 + d, dtype=dtype)
    got = hils.chunk_means(dev(x["K"]))
    torch.cuda.synchronize()
    _means_close(host(got), oracle.chunk_means(x["K"], 64), dtype, "K_lm")


CASES = [
    ("bf16", 1, 2, 2112, 64, 8, False),   # 33 chunks: ragged tiles
    ("bf16", 1, 2, 1024, 128, 16, False),
    ("f32", 1, 2, 1024, 64, 4, False),
    ("bf16", 1, 2, 2112, 64, 8, True),    # with retrieval queries
]


@pytest.mark.parametrize("dtype,B,H,L,d,k,rq", CASES)
def test_fwd_landmark_free(hils, gpu, dtype, B, H, L, d, k, rq):
    say(f"fwd landmark-free dtype={dtype} B={B} H={H} L={L} d={d} k={k} retrieval={rq}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=610 + L + d + rq, dtype=dtype, with_qret=rq)
    t = to_inputs(x, ("Q", "K", "V") + (("Q_ret",) if rq else ()))
    O, idx, sel, w, lse, Klm = hils.sparse_attn_fwd_lf(t["Q"], t["K"], t["V"], k, save_for_backward=True,
                                                       Q_ret=t.get("Q_ret"))
    torch.cuda.synchronize()
    Qr = x["Q_ret"] if rq else None
    ref = oracle.fwd_lf(x["Q"], x["K"], x["V"], 64, k, Q_ret=Qr)
    _means_close(host(Klm), ref["Klm"], dtype, "K_lm")
    gi = idx.cpu().numpy()
    bad = check_selection(gi, ref["idx"], x["Q_ret"] if rq else x["Q"], ref["Klm"], 64, k)
    ro = ref["O"].reshape(-1, d).copy()
    rw = ref["w"].reshape(-1, k + 1).copy()
    ri = ref["idx"].reshape(-1, k + 1).copy()
    if len(bad):
        fix = oracle.fwd_lf(x["Q"], x["K"], x["V"], 64, k, rows=bad, idx=gi.reshape(-1, k + 1)[bad], Q_ret=Qr)
        ro[bad], rw[bad], ri[bad] = fix["O"], fix["w"], fix["idx"]
    assert_close(f32(O).reshape(-1, d), ro, "O", *_tol(dtype))
    # own-slot scores against the causal means
    own = f32(sel).reshape(-1, k + 1)[:, k]
    err = np.abs(own - ref["sel"].reshape(-1, k + 1)[:, k]).max()
    say(f"  own-slot score max err {err:.2e}")
    assert err < 1e-3
    # fusion weights per chunk index
    gw = f32(w).reshape(-1, k + 1)
    gidx = gi.reshape(-1, k + 1)
    for r in range(0, gidx.shape[0], 7):
        gm = {int(j): gw[r, s] for s, j in enumerate(gidx[r]) if j >= 0}
        om = {int(j): rw[r, s] for s, j in enumerate(ri[r]) if j >= 0}
        assert gm.keys() == om.keys()
        for j in gm:
            assert abs(gm[j] - om[j]) < 2e-5, (r, j, gm[j], om[j])


@pytest.mark.parametrize("dtype,B,H,d,ctx,steps,k,rq", [
    ("bf16", 1, 2, 64, 64 * 40 + 10, 70, 4, False),   # crosses a chunk boundary mid-run
    ("bf16", 2, 2, 128, 64 * 300 + 62, 3, 16, True),  # full own chunk, then a fresh one
    ("f32", 1, 2, 64, 64 * 20, 20, 4, False),
])
def test_decode_landmark_free(hils, gpu, dtype, B, H, d, ctx, steps, k, rq):
    say(f"decode landmark-free dtype={dtype} B={B} H={H} d={d} ctx={ctx} steps={steps} k={k} retrieval={rq}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=620 + ctx + d, dtype=dtype, with_qret=rq)
    Lmax = x["K_cache"].shape[2]
    Kc_g, Vc_g = dev(x["K_cache"]), dev(x["V_cache"])
    Kc_h, Vc_h = x["K_cache"].copy(), x["V_cache"].copy()
    # each side forms the landmark rows of the complete chunks itself
    Klm_h = np.zeros_like(x["Klm"])
    oracle.chunk_means(Kc_h, 64, nchunks=ctx // 64, Klm=Klm_h)
    Klm_g = torch.zeros_like(dev(x["Klm"]))
    hils.chunk_means(Kc_g, n_chunks=ctx // 64, K_lm=Klm_g)
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, k), dtype=torch.uint8, device="cuda:0")
    q_all, k_all, v_all = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    qr_all = dev(x["q_ret"]) if rq else None
    tol = _tol(dtype)
    for s in range(steps):
        n = ctx + s
        o, idx, w = hils.decode_step(q_all[s], k_all[s], v_all[s], Kc_g, Vc_g, Klm_g, n, k, ws=ws,
                                     q_ret=qr_all[s] if rq else None, landmark_free=True)
        step = lambda sel=None: oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc_h, Vc_h, Klm_h, n, 64, k,
                                              q_ret=x["q_ret"][s] if rq else None, landmark_free=True,
                                              idx=None if sel is None else sel.reshape(B, H, k + 1))
        ref = step()
        torch.cuda.synchronize()
        gi = idx.cpu().numpy().reshape(B * H, k + 1)
        qs = x["q_ret" if rq else "q"][s].reshape(B * H, d)
        check_decode_step(f"step {s}", gi, f32(w).reshape(B * H, k + 1), f32(o).reshape(B * H, d), ref, step,
                          [n // 64] * (B * H), past_scores_fn(qs, Klm_h.reshape(B * H, -1, d), n // 64, d), k, tol)
    np.testing.assert_array_equal(host(Kc_g), Kc_h)
    # the landmark rows the steps maintained
    last = (ctx + steps - 1) // 64
    _means_close(host(Klm_g)[:, :, :last + 1], Klm_h[:, :, :last + 1], dtype, "K_lm cache")


@pytest.mark.parametrize("dtype,B,H,L,d,k,rq", [
    ("bf16", 1, 2, 2112, 64, 8, False),
    ("bf16", 1, 2, 1024, 128, 16, False),
    ("f32", 1, 2, 1024, 64, 4, False),
    ("f32", 1, 1, 1024, 128, 4, False),
    ("bf16", 1, 2, 2112, 64, 8, True),
])
def test_bwd_landmark_free(hils, gpu, dtype, B, H, L, d, k, rq):
    say(f"bwd landmark-free dtype={dtype} B={B} H={H} L={L} d={d} k={k} retrieval={rq}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=630 + L + d + rq, dtype=dtype, with_dO=True, with_qret=rq)
    t = to_inputs(x, ("Q", "K", "V", "dO") + (("Q_ret",) if rq else ()))
    O, idx, sel, w, lse, Klm = hils.sparse_attn_fwd_lf(t["Q"], t["K"], t["V"], k, save_for_backward=True,
                                                       Q_ret=t.get("Q_ret"))
    grads = hils.sparse_attn_bwd_lf(t["Q"], t["K"], t["V"], Klm, t["dO"], idx, w, lse, k, Q_ret=t.get("Q_ret"))
    torch.cuda.synchronize()
    names = ("dQ", "dQ_ret", "dK", "dV", "dKlm") if rq else ("dQ", "dK", "dV", "dKlm")
    ref = oracle.bwd_lf(x["Q"], x["K"], x["V"], x["dO"], idx.cpu().numpy(), 64, k,
                        Q_ret=x["Q_ret"] if rq else None)
    for name, got in zip(names, grads):
        assert_close(f32(got), ref[name], name, *_tol(dtype))
