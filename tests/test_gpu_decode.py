"""Parity of the HIP decode step with the CPU oracle (and with the prefill path)."""
import numpy as np
import pytest
import torch

import oracle
from long_context_landmark_amd import synth
from gpu_util import GAP, assert_close, check_decode_step, dev, f32, host, say, tol

pytestmark = pytest.mark.gpu


def past_scores_fn(q_h, Klm_h, c, d, scale=None):
    """fp32 scores of row r's past chunks 0..c-1 (double-precision dot products rounded once, as the oracle
    rounds them); q_h [R, d] and Klm_h [R, N, d] in the generated representation."""
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    q64 = synth.as_f32(q_h).astype(np.float64)

    def f(r):
        lm = synth.as_f32(Klm_h[r, :c]).astype(np.float64)
        return (lm @ q64[r] * scale).astype(np.float32)

    return f


def _run_decode(hils, x, k, steps, tol=(2e-2, 1e-2)):
    B, H, Lmax, d = x["K_cache"].shape
    ctx = x["ctx"]
    Kc_g, Vc_g, Klm_g = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
    Kc_h, Vc_h = x["K_cache"].copy(), x["V_cache"].copy()
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, k), dtype=torch.uint8, device="cuda:0")
    q_all, k_all, v_all = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    # optional retrieval queries: they score the landmarks, q keeps the attention
    rq = "q_ret" in x
    qr_all = dev(x["q_ret"]) if rq else None
    Klm_r = x["Klm"].reshape(B * H, -1, d)
    n_differ = 0
    for s in range(steps):
        n = ctx + s
        o, idx, w = hils.decode_step(q_all[s], k_all[s], v_all[s], Kc_g, Vc_g, Klm_g, n, k, ws=ws,
                                     q_ret=qr_all[s] if rq else None)
        step = lambda sel=None: oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc_h, Vc_h, x["Klm"], n, 64,
                                              k, q_ret=x["q_ret"][s] if rq else None,
                                              idx=None if sel is None else sel.reshape(B, H, k + 1))
        ref = step()
        torch.cuda.synchronize()
        gi = idx.cpu().numpy().reshape(B * H, k + 1)
        qs = x["q_ret" if rq else "q"][s].reshape(B * H, d)
        n_differ += check_decode_step(f"step {s}", gi, f32(w).reshape(B * H, k + 1), f32(o).reshape(B * H, d), ref,
                                      step, [n // 64] * (B * H), past_scores_fn(qs, Klm_r, n // 64, d), k, tol)
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
    ("bf16", 1, 3, 64, 64 * 600 + 61, 5, 1),  # top-1: crosses into a fresh chunk, three scan slices
])
def test_decode_steps(hils, gpu, dtype, B, H, d, ctx, steps, k):
    say(f"decode dtype={dtype} B={B} H={H} d={d} ctx={ctx} steps={steps} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=ctx + d, dtype=dtype)
    bar = tol(dtype)
    _run_decode(hils, x, k, steps, tol=bar)


@pytest.mark.parametrize("dtype,B,H,d,ctx,steps,k", [
    ("bf16", 1, 2, 64, 64 * 40 + 10, 70, 4),
    ("bf16", 2, 2, 128, 64 * 300 + 63, 3, 16),
    ("f32", 1, 2, 64, 64 * 20, 20, 4),
])
def test_decode_steps_retrieval_query(hils, gpu, dtype, B, H, d, ctx, steps, k):
    """Decode with a separate retrieval query scoring the landmarks."""
    say(f"decode retrieval query dtype={dtype} B={B} H={H} d={d} ctx={ctx} steps={steps} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, steps, C=64, seed=ctx + d + 7, dtype=dtype, with_qret=True)
    bar = tol(dtype)
    _run_decode(hils, x, k, steps, tol=bar)


def test_decode_equals_prefill_rows(hils, gpu):
    """A decode step at position n gives the prefill output of row n on the same tensors: equal past-chunk
    sets (or sets that differ only on near ties of the oracle's scores) and, where the sets are equal, equal
    outputs within the parity bar."""
    B, H, d, k = 1, 4, 64, 8
    L = 64 * 50
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=77, dtype="bf16", klm="chunkmean")
    Q, K, V, Klm = (dev(x[n]) for n in ("Q", "K", "V", "Klm"))
    O, idx, _, _, _ = hils.sparse_attn_fwd(Q, K, V, Klm, k)
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, L, d, 64, k), dtype=torch.uint8, device="cuda:0")
    Kc, Vc = K.clone(), V.clone()
    differ = 0
    for n in (0, 1, 63, 64, 100, 640, 1000, 2047, 2048, L - 65, L - 1):
        o, di, dw = hils.decode_step(Q[:, :, n].contiguous(), K[:, :, n].contiguous(), V[:, :, n].contiguous(), Kc, Vc,
                                     Klm, n, k, ws=ws)
        torch.cuda.synchronize()
        c = n // 64
        m = min(k, c)
        a = idx[:, :, n].cpu().numpy().reshape(B * H, k + 1)
        b = di.cpu().numpy().reshape(B * H, k + 1)
        assert np.all(a[:, k] == c) and np.all(b[:, k] == c)
        rows = np.arange(B * H) * L + n
        go, po = f32(o).reshape(-1, d), f32(O[:, :, n]).reshape(-1, d)
        for r in range(B * H):
            sa, sb = set(a[r, :m].tolist()), set(b[r, :m].tolist())
            assert len(sa) == m and len(sb) == m
            if sa != sb:
                S = oracle.landmark_scores_rows(x["Q"], x["Klm"], 64, rows[r:r + 1])[0, :c].astype(np.float32)
                mth = np.sort(S)[::-1][m - 1]
                for j in sa ^ sb:
                    assert abs(float(S[j]) - float(mth)) < GAP, (n, r, j)
                differ += 1
            else:
                assert np.max(np.abs(go[r] - po[r])) < 2e-2, (n, r)
    say(f"  rows whose decode and prefill sets differ on near ties: {differ}")


@pytest.mark.timeout(600)
def test_workload_decode_512k(hils, gpu):
    """The 512K decode workload (B=1 H=16 d=64, 524288 cached tokens, k=16, one needle chunk per head):
    256 appended steps, every step checked against the oracle (selection by the gap rule, o and w with the
    GPU's selection held fixed, max-abs and rel-L2); every step keeps the needle chunk."""
    w = synth.WORKLOADS["decode_512k"]
    say(f"workload {w.name}: generating")
    x = synth.workload_inputs(w)
    say("  running 256 steps")
    B, H, Lmax, d = x["K_cache"].shape
    Kc_g, Vc_g, Klm_g = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
    Kc_h, Vc_h = x["K_cache"], x["V_cache"]
    ws = torch.empty(hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, w.k), dtype=torch.uint8, device="cuda:0")
    q_all, k_all, v_all = dev(x["q"]), dev(x["k_new"]), dev(x["v_new"])
    Klm_r = x["Klm"].reshape(B * H, -1, d)
    differ_total = 0
    for s in range(w.steps):
        n = w.L + s
        o, idx, wt = hils.decode_step(q_all[s], k_all[s], v_all[s], Kc_g, Vc_g, Klm_g, n, w.k, ws=ws)
        step = lambda sel=None: oracle.decode(x["q"][s], x["k_new"][s], x["v_new"][s], Kc_h, Vc_h, x["Klm"], n, 64,
                                              w.k, idx=None if sel is None else sel.reshape(B, H, w.k + 1))
        ref = step()
        gi = idx.cpu().numpy().reshape(B * H, w.k + 1)
        differ_total += check_decode_step(f"step {s}", gi, f32(wt).reshape(B * H, w.k + 1),
                                          f32(o).reshape(B * H, d), ref, step, [n // 64] * (B * H),
                                          past_scores_fn(x["q"][s].reshape(B * H, d), Klm_r, n // 64, d), w.k)
        for h in range(H):
            assert int(x["needle_chunk"][0, h]) in gi[h, :w.k].tolist(), (s, h)
    say(f"  rows with near-tie selection differences over all steps: {differ_total}")


@pytest.mark.parametrize("ctx,d,k", [
    (64 * 9000 + 17, 64, 16),    # 36 scan slices: lists beyond the 32nd lane of the merge
    (64 * 16383 + 40, 64, 8),    # 64 scan slices: the library's largest context
])
def test_decode_many_slices(hils, gpu, ctx, d, k):
    """Contexts above 512K tokens, up to the 16384-chunk limit: more than 32 slice lists per head."""
    say(f"decode many slices ctx={ctx} d={d} k={k} slices={(ctx // 64 + 255) // 256}")
    x = synth.decode_inputs(1, 2, d, ctx, 3, C=64, seed=ctx % 1000, dtype="bf16")
    _run_decode(hils, x, k, 3)


@pytest.mark.parametrize("B,H,d,ctx,k", [(1, 2, 64, 64 * 300 + 17, 16), (2, 3, 128, 64 * 40 + 63, 8)])
def test_decode_stale_workspace(hils, gpu, B, H, d, ctx, k):
    """Leftovers in the workspace (every byte 0xff) give the step of a zeroed workspace, bit for bit:
    the slice lists and partial outputs a kernel reads are written earlier in the same step."""
    say(f"decode stale workspace B={B} H={H} d={d} ctx={ctx} k={k}")
    x = synth.decode_inputs(B, H, d, ctx, 1, seed=23)
    Lmax = x["K_cache"].shape[2]
    n = hils.workspace_size(hils.OP_DECODE, B, H, Lmax, d, 64, k)
    res = []
    for fill in (0, 255):
        Kc, Vc, Klm = dev(x["K_cache"]), dev(x["V_cache"]), dev(x["Klm"])
        ws = torch.full((n,), fill, dtype=torch.uint8, device=gpu)
        o, idx, w = hils.decode_step(dev(x["q"])[0], dev(x["k_new"])[0], dev(x["v_new"])[0], Kc, Vc, Klm, ctx, k,
                                     ws=ws)
        res.append((o, idx, w, Kc, Vc))
    for name, a, b in zip(("o", "idx", "w", "K_cache", "V_cache"), *res):
        assert torch.equal(a, b), name
