"""Parity of the several-landmarks-per-chunk forward with the CPU oracle.

A chunk's score is the log-sum-exp of its landmark scores (the HiLS summary page, "Method" >
"Input & chunking" and "Key modules" item 1).  Landmarks: the keys of each chunk's first and last
token, or random rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_landmark_amd import synth
from gpu_util import GAP, assert_close, check_decode_step, dev, f32, say, to_inputs, tol

pytestmark = pytest.mark.gpu


def _landmarks(x, kind, m, seed):
    if kind == "firstlast":
        return synth.first_last_landmarks(x["K"], 64)
    B, H, L, d = x["K"].shape
    lm = np.random.default_rng(seed).standard_normal((B, H, L // 64, m, d), dtype=np.float32)
    return synth.f32_to_bf16_bits(lm) if x["K"].dtype == np.uint16 else lm


def _check_sets(gi, ri, Qs, lm, k):
    """Index sets equal, or differing only where the oracle's chunk scores are within GAP of the m-th best."""
    B, H, L, _ = gi.shape
    d = Qs.shape[-1]
    g, r = gi.reshape(-1, k + 1), ri.reshape(-1, k + 1)
    t_of = np.arange(g.shape[0]) % L
    np.testing.assert_array_equal(g[:, k], t_of // 64)
    bad = []
    for row in range(g.shape[0]):
        c = t_of[row] // 64
        m = min(k, c)
        assert np.all(g[row, m:k] == -1)
        a, b = set(g[row, :m].tolist()), set(r[row, :m].tolist())
        if a == b:
            continue
        bh = row // L
        q = synth.as_f32(Qs.reshape(-1, L, d)[bh, t_of[row]]).astype(np.float64)
        lmf = synth.as_f32(lm.reshape(B * H, lm.shape[2], lm.shape[3], d)[bh, :c]).astype(np.float64)
        a_r = lmf @ q / math.sqrt(d)
        sc = np.log(np.exp(a_r - a_r.max(1, keepdims=True)).sum(1)) + a_r.max(1)
        sc = sc.astype(np.float32)
        mth = np.sort(sc)[::-1][m - 1]
        for j in a ^ b:
            assert abs(float(sc[j]) - float(mth)) < GAP, (row, j)
        bad.append(row)
    say(f"  selection: {len(bad)} of {g.shape[0]} rows differ on near ties")
    return np.asarray(bad, np.int64)


@pytest.mark.parametrize("dtype,B,H,L,d,k,kind,m", [
    ("bf16", 1, 2, 2112, 64, 8, "firstlast", 2),
    ("bf16", 1, 2, 1024, 128, 16, "firstlast", 2),
    ("f32", 1, 2, 1024, 64, 4, "firstlast", 2),
    ("bf16", 1, 2, 2048, 64, 8, "random", 3),
    # 129 chunks: the most that keep both score tiles in registers (query chunks 64 and 128 score
    # their own chunk outside the candidate tiles); from 160 chunks on the sweeps recompute them
    ("bf16", 1, 2, 8256, 64, 4, "random", 2),
    ("bf16", 1, 1, 4160, 128, 16, "random", 3),
    ("f32", 1, 1, 4160, 128, 8, "firstlast", 2),
    ("bf16", 1, 1, 10240, 64, 8, "firstlast", 2),
    # long candidate lists: landmark rows read directly, scores recomputed in each sweep
    ("bf16", 1, 1, 64 * 200, 128, 16, "random", 3),
    ("f32", 1, 1, 64 * 140, 64, 4, "random", 2),
])
def test_fwd_multi_landmark(hils, gpu, dtype, B, H, L, d, k, kind, m):
    say(f"fwd several landmarks dtype={dtype} B={B} H={H} L={L} d={d} k={k} landmarks={kind}x{m}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=800 + L + d + m, dtype=dtype)
    lm = _landmarks(x, kind, m, seed=801 + L)
    t = to_inputs(x, ("Q", "K", "V"))
    O, idx, sel, w, lse = hils.sparse_attn_fwd_ml(t["Q"], t["K"], t["V"], dev(lm), k, save_for_backward=True)
    torch.cuda.synchronize()
    ref = oracle.fwd_ml(x["Q"], x["K"], x["V"], lm, 64, k)
    gi = idx.cpu().numpy()
    bad = _check_sets(gi, ref["idx"], x["Q"], lm, k)
    ro = ref["O"].reshape(-1, d).copy()
    rw = ref["w"].reshape(-1, k + 1).copy()
    ri = ref["idx"].reshape(-1, k + 1).copy()
    if len(bad):
        fix = oracle.fwd_ml(x["Q"], x["K"], x["V"], lm, 64, k, rows=bad, idx=gi.reshape(-1, k + 1)[bad])
        ro[bad], rw[bad], ri[bad] = fix["O"], fix["w"], fix["idx"]
    bar = tol(dtype)
    assert_close(f32(O).reshape(-1, d), ro, "O", *bar)
    gw, gx = f32(w).reshape(-1, k + 1), gi.reshape(-1, k + 1)
    for r in range(0, gx.shape[0], 5):
        gm = {int(j): gw[r, s] for s, j in enumerate(gx[r]) if j >= 0}
        om = {int(j): rw[r, s] for s, j in enumerate(ri[r]) if j >= 0}
        assert gm.keys() == om.keys()
        for j in gm:
            assert abs(gm[j] - om[j]) < 2e-5, (r, j, gm[j], om[j])
    # own-chunk scores
    own = f32(sel).reshape(-1, k + 1)[:, k]
    assert np.abs(own - ref["sel"].reshape(-1, k + 1)[:, k]).max() < 1e-4


@pytest.mark.parametrize("L", [8256, 10240])
def test_fwd_multi_landmark_ties(hils, gpu, L):
    """Every chunk has the same landmarks, so all chunk scores tie and each query keeps the lowest
    indices; with more than 64 tied candidates the survivor list overflows and the exact
    fallback of the selection runs (short lists: over the kept tiles; long ones: recomputed)."""
    B, H, d, k = 1, 1, 64, 8
    say(f"fwd several landmarks, all scores tied, L={L}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=830, dtype="bf16")
    row = np.random.default_rng(831).standard_normal((1, 1, 1, 2, d), dtype=np.float32)
    lm = synth.f32_to_bf16_bits(np.ascontiguousarray(np.broadcast_to(row, (B, H, L // 64, 2, d))))
    t = to_inputs(x, ("Q", "K", "V"))
    O, idx, sel, w, lse = hils.sparse_attn_fwd_ml(t["Q"], t["K"], t["V"], dev(lm), k, save_for_backward=True)
    torch.cuda.synchronize()
    ref = oracle.fwd_ml(x["Q"], x["K"], x["V"], lm, 64, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    assert_close(f32(O), ref["O"], "O (tied scores)", *tol("bf16"))
    assert_close(f32(w), ref["w"], "w (tied scores)", 1e-5, 1e-5)


def test_fwd_multi_landmark_fixed_selection(hils, gpu):
    B, H, L, d, k = 1, 2, 1024, 64, 4
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=810, dtype="bf16")
    lm = synth.first_last_landmarks(x["K"], 64)
    ref = oracle.fwd_ml(x["Q"], x["K"], x["V"], lm, 64, k)
    idx = ref["idx"].copy()
    rng = np.random.default_rng(1)
    for bh in range(B * H):
        for tt in range(L):
            c = tt // 64
            if c > k:
                idx[0, bh, tt, :k] = np.sort(rng.choice(c, size=k, replace=False))
    t = to_inputs(x, ("Q", "K", "V"))
    O, _, sel, w, lse = hils.sparse_attn_fwd_ml(t["Q"], t["K"], t["V"], dev(lm), k, idx=torch.from_numpy(idx).to(gpu),
                                                save_for_backward=True)
    want = oracle.fwd_ml(x["Q"], x["K"], x["V"], lm, 64, k, idx=idx)
    assert_close(f32(O), want["O"], "O (fixed selection)")
    assert_close(f32(w), want["w"], "w (fixed selection)", 1e-5, 1e-5)


@pytest.mark.parametrize("dtype,B,H,L,d,k,kind,m,rq", [
    ("bf16", 1, 2, 2112, 64, 8, "firstlast", 2, False),
    ("bf16", 1, 2, 1024, 128, 16, "firstlast", 2, False),
    ("f32", 1, 2, 1024, 64, 4, "firstlast", 2, False),
    ("bf16", 1, 2, 2048, 64, 8, "random", 3, True),
    ("f32", 1, 1, 1024, 128, 4, "firstlast", 2, False),
])
def test_bwd_multi_landmark(hils, gpu, dtype, B, H, L, d, k, kind, m, rq):
    say(f"bwd several landmarks dtype={dtype} B={B} H={H} L={L} d={d} k={k} landmarks={kind}x{m} retrieval={rq}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=820 + L + d + m, dtype=dtype, with_dO=True, with_qret=rq)
    lm = _landmarks(x, kind, m, seed=821 + L)
    t = to_inputs(x, ("Q", "K", "V", "dO") + (("Q_ret",) if rq else ()))
    lm_g = dev(lm)
    O, idx, sel, w, lse = hils.sparse_attn_fwd_ml(t["Q"], t["K"], t["V"], lm_g, k, save_for_backward=True,
                                                  Q_ret=t.get("Q_ret"))
    grads = hils.sparse_attn_bwd_ml(t["Q"], t["K"], t["V"], lm_g, t["dO"], idx, w, lse, k, Q_ret=t.get("Q_ret"))
    torch.cuda.synchronize()
    ref = oracle.bwd_ml(x["Q"], x["K"], x["V"], lm, x["dO"], idx.cpu().numpy(), 64, k,
                        Q_ret=x["Q_ret"] if rq else None)
    names = ("dQ", "dQ_ret", "dK", "dV", "dKlm") if rq else ("dQ", "dK", "dV", "dKlm")
    bar = tol(dtype)
    for name, got in zip(names, grads):
        assert_close(f32(got), ref[name], name, *bar)


@pytest.mark.parametrize("dtype,H,d,ctx,steps,k,m", [
    ("bf16", 2, 64, 64 * 40 + 10, 70, 4, 2),   # crosses a chunk boundary
    ("bf16", 2, 128, 64 * 300 + 62, 3, 16, 3),  # several scan slices
    ("f32", 2, 64, 64 * 20, 20, 4, 2),
])
def test_decode_multi_landmark(hils, gpu, dtype, H, d, ctx, steps, k, m):
    B = 1
    say(f"decode several landmarks dtype={dtype} H={H} d={d} ctx={ctx} steps={steps} k={k} m={m}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=830 + ctx + d, dtype=dtype)
    Nmax = x["Klm"].shape[2]
    lm = np.random.default_rng(831).standard_normal((B, H, Nmax, m, d), dtype=np.float32)
    lm = synth.f32_to_bf16_bits(lm) if dtype == "bf16" else lm
    Lmax = x["K_cache"].shape[2]
    Kc_g, Vc_g, lm_g = dev(x["K_cache"]), dev(x["V_cache"]), dev(lm)
    Kc_h, Vc_h = x["K_cache"].copy(), x["V_cache"].copy()
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, k), dtype=torch.uint8, device=gpu)
    bar = tol(dtype)
    lmf = synth.as_f32(lm).astype(np.float64)[0]
    for s in range(steps):
        n = ctx + s
        o, idx, w = hils.decode_step(dev(x["q"][s]), dev(x["k_new"][s]), dev(x["v_new"][s]), Kc_g, Vc_g, lm_g, n, k,
                                     ws=ws)
        step = lambda sel=None: oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc_h, Vc_h, lm, n, 64, k,
                                              idx=None if sel is None else sel.reshape(B, H, k + 1))
        ref = step()
        torch.cuda.synchronize()
        c = n // 64

        def past(h, s=s, c=c):
            q = synth.as_f32(x["q"][s][0, h]).astype(np.float64)
            sc_r = lmf[h, :c] @ q / np.sqrt(d)
            return (np.log(np.exp(sc_r - sc_r.max(1, keepdims=True)).sum(1)) + sc_r.max(1)).astype(np.float32)

        check_decode_step(f"step {s}", idx.cpu().numpy().reshape(H, k + 1), f32(w).reshape(H, k + 1),
                          f32(o).reshape(H, d), ref, step, [c] * H, past, k, bar)


@pytest.mark.parametrize("L", [2048, 10240])
def test_multi_landmark_deterministic(hils, gpu, L):
    """Two runs of the several-landmark forward and backward agree bit for bit, with short (tiles kept
    in registers) and long candidate lists, and dq_reduce's landmark terms."""
    B, H, d, k = 1, 2, 64, 8
    say(f"several landmarks, determinism L={L}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=840 + L, dtype="bf16", with_dO=True)
    lm = dev(_landmarks(x, "random", 3, seed=841))
    t = to_inputs(x, ("Q", "K", "V", "dO"))
    runs = []
    for _ in range(2):
        fw = hils.sparse_attn_fwd_ml(t["Q"], t["K"], t["V"], lm, k, save_for_backward=True)
        O, idx, sel, w, lse = fw
        g = hils.sparse_attn_bwd_ml(t["Q"], t["K"], t["V"], lm, t["dO"], idx, w, lse, k)
        torch.cuda.synchronize()
        runs.append(tuple(fw) + tuple(g))
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("L", [8256, 10240])
def test_one_landmark_matches_plain_forward(hils, gpu, L):
    """With m = 1 the chunk score is the landmark score itself: the several-landmark selection picks the
    same chunks as the plain one (the candidate scores come from the same MFMA products), and scores,
    weights and outputs agree to rounding (the own chunk is scored on another unit for some query
    chunks)."""
    B, H, d, k = 1, 2, 64, 8
    say(f"one landmark against the plain forward, L={L}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=850 + L, dtype="bf16")
    t = to_inputs(x, ("Q", "K", "V", "Klm"))
    a = hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, save_for_backward=True)
    b = hils.sparse_attn_fwd_ml(t["Q"], t["K"], t["V"], t["Klm"][:, :, :, None, :].contiguous(), k,
                                save_for_backward=True)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1])
    used = a[1].cpu().numpy() >= 0  # unused slots hold -inf scores in both
    assert np.array_equal(np.isneginf(f32(a[2])), ~used) and np.array_equal(np.isneginf(f32(b[2])), ~used)
    assert np.abs(f32(a[2])[used] - f32(b[2])[used]).max() < 1e-4
    assert np.abs(f32(a[3]) - f32(b[3])).max() < 1e-4
    assert_close(f32(b[0]), f32(a[0]), "O (one landmark against plain)", 1e-2, 1e-3)
