"""Parity of the HIP decode step with the CPU oracle (and with the prefill path)."""
import numpy as np
import pytest
import torch

import oracle
from long_context_landmark_amd import synth
from gpu_util import GAP, assert_close, dev, f32, host, say

pytestmark = pytest.mark.gpu


def _check_step(s, n, g_idx, g_w, g_o, ref, Klm_h, q_h, k, d, C=64, tol=(2e-2, 1e-2)):
    """Selection by the gap rule, then o and w against the oracle (with the GPU selection where sets differ)."""
    B, H = g_idx.shape[:2]
    c = n // C
    m = min(k, c)
    gi = g_idx.reshape(-1, k + 1)
    oi = ref["idx"].reshape(-1, k + 1)
    assert np.all(gi[:, k] == c)
    assert np.all(gi[:, m:k] == -1)
    differ = []
    for bh in range(B * H):
        a, b = set(gi[bh, :m].tolist()), set(oi[bh, :m].tolist())
        if a != b:
            qrow = q_h.reshape(B * H, d)[bh].astype(np.float64) if q_h.dtype != np.uint16 else \
                synth.bf16_bits_to_f32(q_h.reshape(B * H, d)[bh]).astype(np.float64)
            lm = Klm_h.reshape(B * H, -1, d)[bh]
            lmf = synth.bf16_bits_to_f32(lm) if lm.dtype == np.uint16 else lm
            sc = (lmf[:c].astype(np.float64) @ qrow / np.sqrt(d)).astype(np.float32)
            mth = np.sort(sc)[::-1][m - 1]
            for j in a ^ b:
                assert abs(float(sc[j]) - float(mth)) < GAP, (s, bh, j)
            differ.append(bh)
    return differ


def _run_decode(hils, x, k, steps, check_every=1, tol=(2e-2, 1e-2)):
    B, H, Lmax, d = x["K_cache"].shape
    ctx = x["ctx"]
    Kc_g, Vc_g, Klm_g = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
    Kc_h, Vc_h = x["K_cache"].copy(), x["V_cache"].copy()
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, k), dtype=torch.uint8, device="cuda:0")
    q_all, k_all, v_all = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    # optional retrieval queries: they score the landmarks, q keeps the attention
    rq = "q_ret" in x
    qr_all = dev(x["q_ret"]) if rq else None
    n_differ = 0
    for s in range(steps):
        n = ctx + s
        o, idx, w = hils.decode_step(q_all[s], k_all[s], v_all[s], Kc_g, Vc_g, Klm_g, n, k, ws=ws,
                                     q_ret=qr_all[s] if rq else None)
        ref = oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc_h, Vc_h, x["Klm"], n, 64, k,
                            q_ret=x["q_ret"][s] if rq else None)
        if s % check_every and s != steps - 1:
            continue
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        differ = _check_step(s, n, gi, f32(w), f32(o), ref, x["Klm"], x["q_ret" if rq else "q"][s], k, d)
        ro = ref["o"].reshape(B * H, d).copy()
        rw = ref["w"].reshape(B * H, k + 1).copy()
        for bh in differ:
            n_differ += 1
            b, h = divmod(bh, H)
            # oracle forward of this single row with the GPU's selection
            L = ((n // 64) + 1) * 64
            Qp = np.zeros((1, 1, L, d), x["q"].dtype)
            Qp[0, 0, n] = x["q"][s][b, h]
            Qr = None
            if rq:
                Qr = np.zeros_like(Qp)
                Qr[0, 0, n] = x["q_ret"][s][b, h]
            Kp = np.ascontiguousarray(Kc_h[b:b + 1, h:h + 1, :L])
            Vp = np.ascontiguousarray(Vc_h[b:b + 1, h:h + 1, :L])
            Lp = np.ascontiguousarray(x["Klm"][b:b + 1, h:h + 1, :L // 64])
            fx = oracle.fwd(Qp, Kp, Vp, Lp, 64, k, rows=[n], idx=gi.reshape(B * H, k + 1)[bh:bh + 1], Q_ret=Qr)
            ro[bh] = fx["O"][0]
            rw[bh] = fx["w"][0]
        assert_close(f32(o).reshape(B * H, d), ro, f"o step {s}", *tol)
        # weights compared per chunk index
        gw = f32(w).reshape(B * H, k + 1)
        gidx = gi.reshape(B * H, k + 1)
        for bh in range(B * H):
            if bh in differ:
                continue
            gm = {int(j): gw[bh, r] for r, j in enumerate(gidx[bh]) if j >= 0}
            om = {int(j): rw[bh, r] for r, j in enumerate(ref["idx"].reshape(B * H, k + 1)[bh]) if j >= 0}
            assert gm.keys() == om.keys()
            for j in gm:
                assert abs(gm[j] - om[j]) < 1e-5
    # the caches were appended identically
    np.testing.assert_array_equal(host(Kc_g), Kc_h)
    np.testing.assert_array_equal(host(Vc_g), Vc_h)
    say(f"  rows with near-tie selection differences: {n_differ}")
    return Kc_g, Vc_g


@pytest.mark.parametrize("dtype,B,H,d,ctx,steps,k", [
    ("bf16", 1, 2, 64, 64 * 40 + 10, 70, 4),   # crosses a chunk boundary mid-run
    ("bf16", 2, 2, 128, 64 * 300 + 63, 3, 16),  # 3 scan slices, full own chunk, then a fresh chunk
    ("bf16", 1, 3, 64, 5, 64, 8),              # first chunk only, then c = 1
    ("f32", 1, 2, 64, 64 * 20, 20, 4),
    ("f32", 1, 1, 128, 64 * 150 + 7, 4, 16),
])
def test_decode_steps(hils, gpu, dtype, B, H, d, ctx, steps, k):
    say(f"decode dtype={dtype} B={B} H={H} d={d} ctx={ctx} steps={steps} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=ctx + d, dtype=dtype)
    tol = (5e-3, 3e-3) if dtype == "f32" else (2e-2, 1e-2)
    _run_decode(hils, x, k, steps, tol=tol)


@pytest.mark.parametrize("dtype,B,H,d,ctx,steps,k", [
    ("bf16", 1, 2, 64, 64 * 40 + 10, 70, 4),
    ("bf16", 2, 2, 128, 64 * 300 + 63, 3, 16),
    ("f32", 1, 2, 64, 64 * 20, 20, 4),
])
def test_decode_steps_retrieval_query(hils, gpu, dtype, B, H, d, ctx, steps, k):
    """Decode with a separate retrieval query scoring the landmarks."""
    say(f"decode retrieval query dtype={dtype} B={B} H={H} d={d} ctx={ctx} steps={steps} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=ctx + d + 7, dtype=dtype, with_qret=True)
    tol = (5e-3, 3e-3) if dtype == "f32" else (2e-2, 1e-2)
    _run_decode(hils, x, k, steps, tol=tol)


def test_decode_equals_prefill_rows(hils, gpu):
    """A decode step at position n gives the prefill output of row n on the same tensors."""
    B, H, d, k = 1, 2, 64, 8
    L = 64 * 50
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=77, dtype="bf16", klm="chunkmean")
    Q, K, V, Klm = (dev(x[n]) for n in ("Q", "K", "V", "Klm"))
    O, idx, _, _, _ = hils.sparse_attn_fwd(Q, K, V, Klm, k)
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, L, d, 64, k), dtype=torch.uint8, device="cuda:0")
    Kc, Vc = K.clone(), V.clone()
    for n in (0, 1, 63, 64, 100, 640, L - 1):
        o, di, dw = hils.decode_step(Q[:, :, n].contiguous(), K[:, :, n].contiguous(), V[:, :, n].contiguous(), Kc, Vc,
                                     Klm, n, k, ws=ws)
        torch.cuda.synchronize()
        a = np.sort(idx[:, :, n].cpu().numpy(), -1)
        b = np.sort(di.cpu().numpy(), -1)
        same = np.all(a == b, -1).reshape(-1)
        assert same.mean() >= 0.5
        go, po = f32(o).reshape(-1, d), f32(O[:, :, n]).reshape(-1, d)
        assert np.max(np.abs(go[same] - po[same])) < 2e-2


@pytest.mark.timeout(600)
def test_workload_decode_512k(hils, gpu):
    """The 512K decode workload (B=1 H=16 d=64, 524288 cached tokens, k=16, one needle chunk per head):
    256 appended steps, each checked against the oracle; every step keeps the needle chunk."""
    w = synth.WORKLOADS["decode_512k"]
    say(f"workload {w.name}: generating")
    x = synth.workload_inputs(w)
    say("  running 256 steps")
    B, H, Lmax, d = x["K_cache"].shape
    Kc_g, Vc_g, Klm_g = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
    Kc_h, Vc_h = x["K_cache"], x["V_cache"]
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, w.k), dtype=torch.uint8, device="cuda:0")
    q_all, k_all, v_all = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    differ_total = 0
    for s in range(w.steps):
        n = w.L + s
        o, idx, wt = hils.decode_step(q_all[s], k_all[s], v_all[s], Kc_g, Vc_g, Klm_g, n, w.k, ws=ws)
        ref = oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc_h, Vc_h, x["Klm"], n, 64, w.k)
        gi = idx.cpu().numpy()
        differ = _check_step(s, n, gi, f32(wt), f32(o), ref, x["Klm"], x["q"][s], w.k, d)
        differ_total += len(differ)
        keep = np.ones(B * H, bool)
        keep[differ] = False
        assert_close(f32(o).reshape(B * H, d)[keep], ref["o"].reshape(B * H, d)[keep], f"o step {s}") if s % 32 == 0 \
            else None
        go = f32(o).reshape(B * H, d)[keep]
        ma = np.max(np.abs(go - ref["o"].reshape(B * H, d)[keep]))
        assert ma < 2e-2, (s, ma)
        for h in range(H):
            assert int(x["needle_chunk"][0, h]) in gi[0, h, :w.k].tolist(), (s, h)
    say(f"  rows with near-tie selection differences over all steps: {differ_total}")
