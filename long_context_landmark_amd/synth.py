"""Seeded synthetic inputs for HiLS attention.

This module builds operator *inputs* only: it holds none of the operator's
arithmetic (no scores, no selection, no attention).  Both sides of every parity
check -- the HIP library and the CPU oracle -- receive the same bytes from here.

Recipe (the stand-in for the pages' long-context workloads; the evaluation
suites themselves are not available and are not reproduced):
  * ``numpy.random.default_rng(seed)``; draw order Q, K, V, landmark noise,
    needle choices, decode per-step draws, dO, retrieval-query noise.  Each
    draw is float32 ``standard_normal`` of the full shape in C order, then
    scaled.
  * retrieval queries (optional, for the low-rank query calibration of the
    "Method" section's input stage): Q_ret = 0.6 Q + 0.8 n, n a fresh
    standard-normal draw of Q's shape, formed in float32 from Q before Q is
    rounded, so Q_ret is correlated with Q but not equal to it.
  * bf16 tensors are rounded from float32 with round-to-nearest-even and are
    carried on the host as uint16 bit patterns.
  * ``klm="chunkmean"``: each landmark row is the mean of its chunk's keys
    (taken from the already-rounded keys) plus N(0, klm_noise^2).
  * needles: for each (b,h) one unit direction u; each needle chunk's landmark
    becomes ||Klm_n|| u, and each designated query is rotated to
    ||q|| (0.9 u + sqrt(0.19) v) with v its unit component orthogonal to u,
    so cos(q, Klm_n) = 0.9 exactly before rounding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Values of a generated tensor as float32 (bf16 bits are widened exactly)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, np.float32)


def _unit(rng, shape_lead, d):
    u = rng.standard_normal(shape_lead + (d,), dtype=np.float32).astype(np.float64)
    return u / np.linalg.norm(u, axis=-1, keepdims=True)


def _align(x: np.ndarray, u: np.ndarray, cos: float = 0.9) -> np.ndarray:
    """Rotate rows of x (float64 [..., d]) to cosine ``cos`` with unit u [..., d], keeping their norm."""
    nx = np.linalg.norm(x, axis=-1, keepdims=True)
    par = np.sum(x * u, axis=-1, keepdims=True)
    perp = x - par * u
    perp /= np.maximum(np.linalg.norm(perp, axis=-1, keepdims=True), 1e-30)
    return nx * (cos * u + math.sqrt(1.0 - cos * cos) * perp)


def prefill_inputs(B, H, L, d, C=64, seed=0, dtype="bf16", qkv_std=1.0, klm="iid", klm_noise=0.1,
                   needles=0, needle_window=256, with_dO=False, with_qret=False):
    """Inputs of one prefill (or training) call.

    Returns a dict with Q, K, V [B,H,L,d], Klm [B,H,N,d] (uint16 bf16 bits or
    float32), optionally dO, and ``needle_chunks`` [B,H,needles] int64.
    """
    if L % C:
        raise ValueError("L must be a multiple of C")
    N = L // C
    rng = np.random.default_rng(seed)
    shp = (B, H, L, d)
    Q = rng.standard_normal(shp, dtype=np.float32) * np.float32(qkv_std)
    K = _finish(rng.standard_normal(shp, dtype=np.float32) * np.float32(qkv_std), dtype)
    V = _finish(rng.standard_normal(shp, dtype=np.float32) * np.float32(qkv_std), dtype)
    noise = rng.standard_normal((B, H, N, d), dtype=np.float32)
    if klm == "iid":
        Klm = noise.astype(np.float64)
    elif klm == "chunkmean":
        Kf = as_f32(K).astype(np.float64).reshape(B, H, N, C, d)
        Klm = Kf.mean(axis=3) + klm_noise * noise.astype(np.float64)
    else:
        raise ValueError(klm)
    needle_chunks = np.zeros((B, H, needles), np.int64)
    if needles:
        first_q = L - needle_window
        hi = first_q // C  # needle chunks are past chunks for every designated query
        u = _unit(rng, (B, H), d)
        for b in range(B):
            for h in range(H):
                needle_chunks[b, h] = rng.choice(hi, size=needles, replace=False)
        Qd = Q.astype(np.float64)
        for b in range(B):
            for h in range(H):
                for n in needle_chunks[b, h]:
                    Klm[b, h, n] = np.linalg.norm(Klm[b, h, n]) * u[b, h]
                Qd[b, h, first_q:] = _align(Qd[b, h, first_q:], u[b, h][None, :])
        Q = Qd.astype(np.float32)
    out = {
        "Q": _finish(Q, dtype),
        "K": K,
        "V": V,
        "Klm": _finish(Klm.astype(np.float32), dtype),
        "needle_chunks": needle_chunks,
    }
    if with_dO:
        out["dO"] = _finish(rng.standard_normal(shp, dtype=np.float32), dtype)
    if with_qret:
        out["Q_ret"] = _retrieval(rng, Q, dtype)
    return out


def _retrieval(rng, q, dtype):
    n = rng.standard_normal(q.shape, dtype=np.float32)
    return _finish(np.float32(0.6) * q.astype(np.float32) + np.float32(0.8) * n, dtype)


def decode_inputs(B, H, d, ctx, steps, C=64, seed=0, dtype="bf16", needle=True, with_qret=False):
    """Inputs of a decode run: caches filled to ``ctx`` rows, then ``steps`` new tokens.

    Returns K_cache, V_cache [B,H,Lmax,d] (rows >= ctx zero until appended),
    Klm [B,H,Nmax,d] (every row drawn up front; the row of a chunk is the
    caller-supplied landmark of that chunk from the step that opens it),
    q, k_new, v_new [steps,B,H,d] and ``needle_chunk`` [B,H].
    """
    Lmax = ctx + steps
    Nmax = (Lmax + C - 1) // C
    rng = np.random.default_rng(seed)
    Kc = np.zeros((B, H, Lmax, d), np.float32)
    Vc = np.zeros((B, H, Lmax, d), np.float32)
    Kc[:, :, :ctx] = rng.standard_normal((B, H, ctx, d), dtype=np.float32)
    Vc[:, :, :ctx] = rng.standard_normal((B, H, ctx, d), dtype=np.float32)
    Klm = rng.standard_normal((B, H, Nmax, d), dtype=np.float32).astype(np.float64)
    nch = np.zeros((B, H), np.int64)
    u = None
    needle = needle and ctx // C > 0
    if needle:
        u = _unit(rng, (B, H), d)
        nch = rng.integers(0, ctx // C, size=(B, H))
        for b in range(B):
            for h in range(H):
                Klm[b, h, nch[b, h]] = np.linalg.norm(Klm[b, h, nch[b, h]]) * u[b, h]
    q = rng.standard_normal((steps, B, H, d), dtype=np.float32).astype(np.float64)
    k_new = rng.standard_normal((steps, B, H, d), dtype=np.float32)
    v_new = rng.standard_normal((steps, B, H, d), dtype=np.float32)
    if needle:
        q = _align(q, u[None])
    out = {
        "K_cache": _finish(Kc, dtype),
        "V_cache": _finish(Vc, dtype),
        "Klm": _finish(Klm.astype(np.float32), dtype),
        "q": _finish(q.astype(np.float32), dtype),
        "k_new": _finish(k_new, dtype),
        "v_new": _finish(v_new, dtype),
        "needle_chunk": nch,
        "ctx": ctx,
    }
    if with_qret:
        out["q_ret"] = _retrieval(rng, q, dtype)
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "decode" | "train"
    B: int
    H: int
    d: int
    L: int  # sequence length (prefill/train) or cached context (decode)
    k: int
    C: int = 64
    dtype: str = "bf16"
    seed: int = 0
    gen: dict = field(default_factory=dict)
    steps: int = 0


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "prefill", 1, 2, 64, 1024, 4, dtype="f32", seed=1001,
                          gen={"klm": "iid"}),
    "prefill_8k": Workload("prefill_8k", "prefill", 1, 16, 64, 8192, 8, seed=1002,
                           gen={"klm": "chunkmean", "klm_noise": 0.1, "needles": 4, "needle_window": 256}),
    "decode_512k": Workload("decode_512k", "decode", 1, 16, 64, 524288, 16, seed=1003, steps=256),
    "prefill_128k": Workload("prefill_128k", "prefill", 1, 32, 128, 131072, 16, seed=1004,
                             gen={"klm": "chunkmean", "klm_noise": 0.1, "qkv_std": 1.0 / math.sqrt(2.0)}),
    "train_8k": Workload("train_8k", "train", 4, 16, 64, 8192, 8, seed=1005,
                         gen={"klm": "iid", "with_dO": True}),
    # serving shape: 16 sequences with contexts spread over 16K..128K tokens (L = the longest), pages of one
    # chunk in a shuffled pool
    "decode_paged_b16": Workload("decode_paged_b16", "decode", 16, 16, 64, 131072, 16, seed=1006, steps=64,
                                 gen={"ctx_lo": 16384}),
}


def workload_inputs(w: Workload, **override):
    """Host inputs of a named workload (sizes may be overridden, e.g. for a reduced test)."""
    p = dict(B=w.B, H=w.H, d=w.d, C=w.C, seed=w.seed, dtype=w.dtype)
    p.update(override)
    if w.kind == "decode":
        return decode_inputs(p["B"], p["H"], p["d"], override.get("ctx", w.L), override.get("steps", w.steps),
                             C=p["C"], seed=p["seed"], dtype=p["dtype"])
    g = dict(w.gen)
    for key in ("klm", "klm_noise", "needles", "needle_window", "qkv_std", "with_dO"):
        if key in override:
            g[key] = override[key]
    return prefill_inputs(p["B"], p["H"], override.get("L", w.L), p["d"], C=p["C"], seed=p["seed"],
                          dtype=p["dtype"], **g)


# ----------------------------------------------------------------------------
# Device-side generation with torch's seeded RNG, for the benchmark's large
# inputs.  Same recipe as above; the random stream is torch's, not numpy's, so
# values differ from the host generator for the same seed.


def _torch_gen(seed, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def torch_prefill_inputs(w: Workload, device="cuda:0", seed=None, with_dO=None, with_qret=False):
    """Inputs of a prefill / training workload generated on the device (torch tensors)."""
    import torch

    g = _torch_gen(w.seed if seed is None else seed, device)
    B, H, L, d, C = w.B, w.H, w.L, w.d, w.C
    N = L // C
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    std = float(w.gen.get("qkv_std", 1.0))

    def normal(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    Q = normal((B, H, L, d)) * std
    K = (normal((B, H, L, d)) * std).to(dt)
    V = (normal((B, H, L, d)) * std).to(dt)
    noise = normal((B, H, N, d))
    if w.gen.get("klm", "iid") == "chunkmean":
        Klm = K.float().view(B, H, N, C, d).mean(dim=3) + float(w.gen.get("klm_noise", 0.1)) * noise
    else:
        Klm = noise
    needles = int(w.gen.get("needles", 0))
    if needles:
        first_q = L - int(w.gen.get("needle_window", 256))
        u = normal((B, H, d))
        u = u / u.norm(dim=-1, keepdim=True)
        for b in range(B):
            for h in range(H):
                ch = torch.randperm(first_q // C, generator=g, device=device)[:needles]
                Klm[b, h, ch] = Klm[b, h, ch].norm(dim=-1, keepdim=True) * u[b, h]
        q = Q[:, :, first_q:].double()
        uu = u[:, :, None, :].double()
        par = (q * uu).sum(-1, keepdim=True)
        perp = q - par * uu
        perp = perp / perp.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        Q[:, :, first_q:] = (q.norm(dim=-1, keepdim=True) * (0.9 * uu + math.sqrt(0.19) * perp)).float()
    out = {"Q": Q.to(dt).contiguous(), "K": K.contiguous(), "V": V.contiguous(), "Klm": Klm.to(dt).contiguous()}
    if with_dO if with_dO is not None else w.gen.get("with_dO", False):
        out["dO"] = normal((B, H, L, d)).to(dt)
    if with_qret:
        out["Q_ret"] = (0.6 * Q + 0.8 * normal((B, H, L, d))).to(dt).contiguous()
    return out


def torch_decode_inputs(w: Workload, replicas=1, device="cuda:0", seed=None):
    """Decode workload on the device: ``replicas`` independent caches (one per emulated layer) and the
    per-step q, k_new, v_new shared by them.  One needle chunk per head and replica."""
    import torch

    g = _torch_gen(w.seed if seed is None else seed, device)
    B, H, d, C, ctx, steps = w.B, w.H, w.d, w.C, w.L, w.steps
    Lmax = ctx + steps
    Nmax = (Lmax + C - 1) // C
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    reps = []
    u = torch.randn((B, H, d), generator=g, device=device)
    u = u / u.norm(dim=-1, keepdim=True)
    for _ in range(replicas):
        Kc = torch.zeros((B, H, Lmax, d), dtype=dt, device=device)
        Vc = torch.zeros((B, H, Lmax, d), dtype=dt, device=device)
        Kc[:, :, :ctx] = torch.randn((B, H, ctx, d), generator=g, device=device).to(dt)
        Vc[:, :, :ctx] = torch.randn((B, H, ctx, d), generator=g, device=device).to(dt)
        Klm = torch.randn((B, H, Nmax, d), generator=g, device=device)
        nch = torch.randint(0, ctx // C, (B, H), generator=g, device=device)
        for b in range(B):
            for h in range(H):
                j = int(nch[b, h])
                Klm[b, h, j] = Klm[b, h, j].norm() * u[b, h]
        reps.append({"K_cache": Kc, "V_cache": Vc, "Klm": Klm.to(dt).contiguous(), "needle_chunk": nch})
    q = torch.randn((steps, B, H, d), generator=g, device=device).double()
    uu = u[None].double()
    par = (q * uu).sum(-1, keepdim=True)
    perp = q - par * uu
    perp = perp / perp.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    q = q.norm(dim=-1, keepdim=True) * (0.9 * uu + math.sqrt(0.19) * perp)
    k_new = torch.randn((steps, B, H, d), generator=g, device=device).to(dt)
    v_new = torch.randn((steps, B, H, d), generator=g, device=device).to(dt)
    return {"replicas": reps, "q": q.to(dt).contiguous(), "k_new": k_new.contiguous(), "v_new": v_new.contiguous(),
            "ctx": ctx}


def torch_paged_decode_inputs(w: Workload, device="cuda:0", seed=None):
    """Paged decode workload on the device: contexts evenly spread over [ctx_lo, L] (ragged), every chunk a
    pool page in shuffled order (spare pages for the steps), per-step positions, q, k_new and v_new."""
    import torch

    g = _torch_gen(w.seed if seed is None else seed, device)
    B, H, d, C, steps = w.B, w.H, w.d, w.C, w.steps
    lo = int(w.gen.get("ctx_lo", w.L // 2))
    ctx = [lo + (w.L - lo) * b // max(1, B - 1) - (b * 37) % C for b in range(B)]
    nch = [(c + steps - 1) // C + 1 for c in ctx]
    maxp = max(nch)
    P = sum(nch)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    order = torch.randperm(P, generator=g, device=device).to(torch.int32)
    table = torch.zeros((B, maxp), dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        table[b, :nch[b]] = order[off:off + nch[b]]
        off += nch[b]
    Kp = torch.randn((P, H, C, d), generator=g, device=device).to(dt)
    Vp = torch.randn((P, H, C, d), generator=g, device=device).to(dt)
    Lp = torch.randn((P, H, d), generator=g, device=device).to(dt)
    pos = torch.tensor([[c + s for c in ctx] for s in range(steps)], dtype=torch.int64, device=device)
    q = torch.randn((steps, B, H, d), generator=g, device=device).to(dt)
    k_new = torch.randn((steps, B, H, d), generator=g, device=device).to(dt)
    v_new = torch.randn((steps, B, H, d), generator=g, device=device).to(dt)
    return {"K_pages": Kp, "V_pages": Vp, "K_lm_pages": Lp, "page_table": table, "pos": pos,
            "pos_max": [max(ctx) + s for s in range(steps)], "ctx": ctx, "q": q, "k_new": k_new, "v_new": v_new}


def first_last_landmarks(K: np.ndarray, C: int = 64) -> np.ndarray:
    """Two landmarks per chunk, the keys of its first and last token: [B,H,N,2,d] from K [B,H,L,d]
    (a copy of rows, same element type)."""
    B, H, L, d = K.shape
    Kc = K.reshape(B, H, L // C, C, d)
    return np.ascontiguousarray(np.stack([Kc[:, :, :, 0], Kc[:, :, :, C - 1]], axis=3))
