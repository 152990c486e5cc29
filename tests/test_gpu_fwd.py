"""Parity of the HIP prefill path (scores, selection, forward) with the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from long_context_landmark_amd import synth
from gpu_util import assert_close, check_selection, dev, f32, host, say, to_inputs, tol

pytestmark = pytest.mark.gpu


def _inputs(B, H, L, d, k, seed, dtype="bf16", **kw):
    return synth.prefill_inputs(B, H, L, d, C=64, seed=seed, dtype=dtype, **kw)


@pytest.mark.parametrize("dtype,d,L", [("bf16", 64, 1024), ("bf16", 128, 4160), ("f32", 64, 1024), ("f32", 128, 256)])
def test_landmark_scores(hils, gpu, dtype, d, L):
    say(f"landmark_scores dtype={dtype} d={d} L={L}")
    x = _inputs(1, 2, L, d, 4, seed=100 + d, dtype=dtype)
    t = to_inputs(x)
    S = f32(hils.landmark_scores(t["Q"], t["Klm"]))
    ref = oracle.landmark_scores(x["Q"], x["Klm"], 64)
    np.testing.assert_array_equal(np.isneginf(S), np.isneginf(ref))
    ok = np.isfinite(ref)
    err = np.max(np.abs(S[ok] - ref[ok]))
    say(f"  max score error {err:.3e}")
    assert err < (1e-5 if dtype == "f32" else 1e-4)


CASES = [
    # dtype, B, H, L, d, k, klm
    ("bf16", 1, 2, 2048, 64, 4, "iid"),
    ("bf16", 2, 3, 4160, 128, 16, "chunkmean"),  # 65 chunks: ragged landmark tile, partial pair tiles
    ("bf16", 1, 2, 8192, 64, 8, "chunkmean"),
    ("bf16", 1, 1, 64, 64, 4, "iid"),  # single chunk: own chunk only
    ("bf16", 1, 2, 320, 128, 8, "iid"),  # c <= k everywhere: every past chunk kept
    ("bf16", 1, 1, 1024, 64, 16, "iid"),  # k = N
    ("f32", 1, 2, 1024, 64, 4, "iid"),  # the tiny fp32 workload
    ("f32", 1, 1, 2048, 128, 8, "iid"),
    ("bf16", 1, 2, 19200, 64, 16, "iid"),  # 300 chunks: the multi-tile two-sweep selection
    ("bf16", 1, 1, 12352, 128, 8, "chunkmean"),  # 193 chunks, d=128
    ("bf16", 1, 2, 64 * 129, 64, 16, "iid"),  # 129 chunks: the largest short-list selection, m up to 16
    ("bf16", 1, 2, 64 * 130, 64, 8, "chunkmean"),  # 130 chunks: the long-list selection with three tiles
    ("bf16", 1, 3, 4096, 64, 1, "iid"),  # top-1, three heads (no XCD remap)
    ("bf16", 3, 1, 2048, 128, 1, "chunkmean"),  # top-1 at d = 128, three sequences
    # k not a power of two: the routing's pair indices (query t, slot r) of f = t k + r
    ("bf16", 1, 2, 4096, 64, 5, "iid"),
    ("bf16", 2, 1, 64 * 96, 128, 12, "chunkmean"),
    ("bf16", 1, 1, 64 * 300, 64, 7, "iid"),  # 300 chunks: counts scanned apart, staged scatter
]


@pytest.mark.parametrize("dtype,B,H,L,d,k,klm", CASES)
def test_topk_select(hils, gpu, dtype, B, H, L, d, k, klm):
    say(f"topk_select dtype={dtype} B={B} H={H} L={L} d={d} k={k}")
    x = _inputs(B, H, L, d, k, seed=7 + L + d + k, dtype=dtype, klm=klm)
    t = to_inputs(x)
    idx, sel, w = hils.topk_select(t["Q"], t["Klm"], k)
    torch.cuda.synchronize()
    ref = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k)
    gi = idx.cpu().numpy()
    bad = check_selection(gi, ref["idx"], x["Q"], x["Klm"], 64, k)
    same = np.ones(gi.reshape(-1, k + 1).shape[0], bool)
    same[bad] = False
    gsel = f32(sel).reshape(-1, k + 1)[same]
    gw = f32(w).reshape(-1, k + 1)[same]
    order_g = np.argsort(gi.reshape(-1, k + 1)[same], axis=1, kind="stable")
    order_o = np.argsort(ref["idx"].reshape(-1, k + 1)[same], axis=1, kind="stable")
    rs = ref["sel"].reshape(-1, k + 1)[same]
    rw = ref["w"].reshape(-1, k + 1)[same]
    a = np.take_along_axis(gsel, order_g, 1)
    b = np.take_along_axis(rs, order_o, 1)
    fin = np.isfinite(b)
    np.testing.assert_array_equal(np.isfinite(a), fin)
    assert np.max(np.abs(a[fin] - b[fin])) < 1e-4
    assert_close(np.take_along_axis(gw, order_g, 1), np.take_along_axis(rw, order_o, 1), "w", 1e-5, 1e-5)


@pytest.mark.parametrize("d,N,k", [(64, 200, 8), (128, 200, 8), (64, 100, 8), (128, 120, 16)])
def test_topk_exact_ties_fallback(hils, gpu, d, N, k):
    """All landmarks equal: every candidate ties, the survivor buffer overflows and the exact fallback must
    return the m lowest chunk indices (N <= 129 takes the short-sequence kernel)."""
    say(f"topk ties d={d} N={N} k={k}")
    L = 64 * N
    x = _inputs(1, 1, L, d, k, seed=3, klm="iid")
    Klm = np.broadcast_to(x["Klm"][:, :, :1], x["Klm"].shape).copy()
    idx, sel, w = hils.topk_select(dev(x["Q"]), dev(Klm), k)
    gi = idx.cpu().numpy()[0, 0]
    for t in range(0, L, 37):
        c = t // 64
        m = min(k, c)
        assert gi[t, :m].tolist() == list(range(m)), (t, gi[t])
        assert np.all(gi[t, m:k] == -1) and gi[t, k] == c


@pytest.mark.parametrize("dtype,B,H,L,d,k,klm", CASES)
def test_sparse_attn_fwd(hils, gpu, dtype, B, H, L, d, k, klm):
    say(f"sparse_attn_fwd dtype={dtype} B={B} H={H} L={L} d={d} k={k}")
    x = _inputs(B, H, L, d, k, seed=11 + L + d + k, dtype=dtype, klm=klm)
    t = to_inputs(x)
    O, idx, sel, w, lse = hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, save_for_backward=True)
    torch.cuda.synchronize()
    ref = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k)
    gi = idx.cpu().numpy()
    bad = check_selection(gi, ref["idx"], x["Q"], x["Klm"], 64, k)
    go = f32(O).reshape(-1, d)
    ro = ref["O"].reshape(-1, d).copy()
    rl = ref["lse"].reshape(-1, k + 1).copy()
    ri = ref["idx"].reshape(-1, k + 1).copy()
    if len(bad):
        fix = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k, rows=bad, idx=gi.reshape(-1, k + 1)[bad])
        ro[bad] = fix["O"]
        rl[bad] = fix["lse"]
        ri[bad] = fix["idx"]
    # fp32 inputs keep fp32 MFMA arithmetic, but the per-pair partials travel as bf16
    bar = tol(dtype)
    assert_close(go, ro, "O", *bar)
    # per-slot log-partition functions, compared per chunk index
    gl = f32(lse).reshape(-1, k + 1)
    gidx = gi.reshape(-1, k + 1)
    for r in range(0, gidx.shape[0], max(1, gidx.shape[0] // 512)):
        gmap = {int(j): gl[r, s] for s, j in enumerate(gidx[r]) if j >= 0}
        rmap = {int(j): rl[r, s] for s, j in enumerate(ri[r]) if j >= 0}
        assert gmap.keys() == rmap.keys()
        for j in gmap:
            assert abs(gmap[j] - rmap[j]) < 2e-3, (r, j, gmap[j], rmap[j])


def test_fwd_fixed_selection(hils, gpu):
    """select=0: the caller's selection is used as given."""
    B, H, L, d, k = 1, 2, 2048, 64, 4
    say(f"fixed selection B={B} H={H} L={L} d={d} k={k}")
    x = _inputs(B, H, L, d, k, seed=21)
    t = to_inputs(x)
    ref = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k)
    # a selection the scores would not make: reverse the oracle's order and drop the best chunk where possible
    idx = ref["idx"].copy()
    rng = np.random.default_rng(0)
    for bh in range(B * H):
        for tt in range(L):
            c = tt // 64
            m = min(k, c)
            if c > k:
                idx[0, bh, tt, :m] = np.sort(rng.choice(c, size=m, replace=False))
    gidx = torch.from_numpy(idx).to(gpu)
    O, _, sel, w, lse = hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, idx=gidx, save_for_backward=True)
    want = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k, idx=idx)
    assert_close(f32(O), want["O"], "O (fixed selection)")
    assert_close(f32(w), want["w"], "w (fixed selection)", 1e-5, 1e-5)


@pytest.mark.parametrize("H,L,d,k", [(4, 4096, 128, 16), (2, 19200, 64, 16)])  # one- and two-pass routing
def test_fwd_deterministic(hils, gpu, H, L, d, k):
    B = 1
    say(f"determinism B={B} H={H} L={L} d={d} k={k}")
    x = _inputs(B, H, L, d, k, seed=5, klm="chunkmean")
    t = to_inputs(x)
    outs = [hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, save_for_backward=True) for _ in range(2)]
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("H,L,d,k", [(2, 320, 64, 4), (2, 4160, 128, 16), (1, 8192, 64, 8)])
def test_fwd_stale_workspace(hils, gpu, H, L, d, k):
    """A workspace full of leftovers (every byte 0xff) gives the results of a zeroed one, bit for bit:
    every workspace word a kernel reads (routing counts and lists, work items, partial rows) is
    written earlier in the same call.  L = 320 and 4160 leave a partial last routing segment."""
    say(f"stale workspace H={H} L={L} d={d} k={k}")
    x = _inputs(1, H, L, d, k, seed=7, klm="chunkmean")
    t = to_inputs(x)
    n = hils.workspace_size(hils.OP_FWD, 1, H, L, d, 64, k)
    outs = []
    for fill in (0, 255):
        ws = torch.full((n,), fill, dtype=torch.uint8, device=gpu)
        outs.append(hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, save_for_backward=True, ws=ws))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_workload_prefill_8k_full(hils, gpu):
    """The 8K prefill workload (B=1 H=16 d=64 L=8192 k=8, chunk-mean landmarks, 4 needles): every row."""
    w = synth.WORKLOADS["prefill_8k"]
    say(f"workload {w.name}: full parity")
    x = synth.workload_inputs(w)
    t = to_inputs(x)
    O, idx, sel, wt, lse = hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], w.k, save_for_backward=True)
    torch.cuda.synchronize()
    ref = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, w.k)
    gi = idx.cpu().numpy()
    bad = check_selection(gi, ref["idx"], x["Q"], x["Klm"], 64, w.k)
    ro = ref["O"].reshape(-1, w.d).copy()
    if len(bad):
        ro[bad] = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, w.k, rows=bad,
                             idx=gi.reshape(-1, w.k + 1)[bad])["O"]
    assert_close(f32(O).reshape(-1, w.d), ro, "O")
    # every designated query keeps all four needle chunks
    for h in range(w.H):
        needles = set(int(n) for n in x["needle_chunks"][0, h])
        for tq in range(w.L - 256, w.L):
            assert needles <= set(gi[0, h, tq, :w.k].tolist())


@pytest.mark.timeout(400)
def test_workload_prefill_128k_sampled(hils, gpu):
    """The 128K prefill workload (B=1 H=32 d=128 L=131072 k=16) in the launch configuration the benchmark
    times, checked on sampled rows of two heads including chunk boundaries."""
    w = synth.WORKLOADS["prefill_128k"]
    say(f"workload {w.name}: sampled parity")
    x = synth.workload_inputs(w)
    t = to_inputs(x)
    del x["K"], x["V"]
    O, idx, sel, wt, lse = hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], w.k, save_for_backward=True)
    torch.cuda.synchronize()
    heads = [0, 31]
    rng = np.random.default_rng(0)
    ts = np.unique(np.concatenate([rng.integers(0, w.L, 2000), np.arange(0, w.L, 64 * 97), np.arange(63, w.L, 64 * 89),
                                   [0, 1, 63, 64, 1023, 1024, w.L - 1]]))
    # host copies of the sampled heads only
    Kh = host(t["K"][:, heads]).copy()
    Vh = host(t["V"][:, heads]).copy()
    Qh = np.ascontiguousarray(x["Q"][:, heads])
    Lh = np.ascontiguousarray(x["Klm"][:, heads])
    rows = np.concatenate([hi * w.L + ts for hi in range(len(heads))])
    ref = oracle.fwd(Qh, Kh, Vh, Lh, 64, w.k, rows=rows)
    gi = idx[:, heads].cpu().numpy().reshape(-1, w.k + 1)[rows]
    bad = check_selection(gi, ref["idx"], Qh, Lh, 64, w.k, rows=rows)
    ro = ref["O"].copy()
    if len(bad):
        ro[bad] = oracle.fwd(Qh, Kh, Vh, Lh, 64, w.k, rows=rows[bad], idx=gi[bad])["O"]
    go = f32(O[:, heads]).reshape(-1, w.d)[rows]
    assert_close(go, ro, "O (sampled)")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("N,d,k", [(2304, 64, 8), (4100, 128, 16), (16384, 64, 4)])  # 16384: the largest accepted
def test_fwd_beyond_2048_chunks_sampled(hils, gpu, N, d, k):
    """More than 2048 chunks per sequence (the routing's one-wavefront scatter, long top-k candidate lists):
    sampled rows including chunk boundaries against the oracle, and two runs bitwise equal."""
    B, H, L = 1, 1, 64 * N
    say(f"long prefill B={B} H={H} L={L} d={d} k={k} (N={N})")
    x = _inputs(B, H, L, d, k, seed=N + d, klm="chunkmean")
    t = to_inputs(x)
    outs = [hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, save_for_backward=True) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    O, idx = outs[0][0], outs[0][1]
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([rng.integers(0, L, 1500), np.arange(63, L, 64 * 101), [0, 64, 65, L - 64, L - 1],
                                     np.arange(2048 * 64, L, 64 * 37)]))
    ref = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k, rows=rows)
    gi = idx.cpu().numpy().reshape(-1, k + 1)[rows]
    bad = check_selection(gi, ref["idx"], x["Q"], x["Klm"], 64, k, rows=rows)
    ro = ref["O"].copy()
    if len(bad):
        ro[bad] = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k, rows=rows[bad], idx=gi[bad])["O"]
    assert_close(f32(O).reshape(-1, d)[rows], ro, "O (sampled)")
