"""Seeded random shapes through the C ABI: forward and backward against the oracle over mixed batch,
heads, sequence length (any multiple of 64, so ragged pair tiles and partial routing segments),
head size, top-k and input type.  Selection sets follow the gap rule; outputs, fusion weights and
gradients are compared with the oracle run on the GPU's selection."""
import numpy as np
import pytest

import oracle
from long_context_landmark_amd import synth
from gpu_util import assert_close, check_selection, dev, f32, say, to_inputs, tol

pytestmark = pytest.mark.gpu


def _cases(n=10, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if rng.random() < 0.3 else "bf16"
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N, k = int(rng.integers(1, 71)), int(rng.integers(1, 17))
        out.append((i, dtype, B, H, 64 * N, d, k))
    return out


@pytest.mark.parametrize("i,dtype,B,H,L,d,k", _cases())
def test_random_shape_fwd_bwd(hils, gpu, i, dtype, B, H, L, d, k):
    say(f"random shape {i}: dtype={dtype} B={B} H={H} L={L} d={d} k={k}")
    x = synth.prefill_inputs(B, H, L, d, C=64, seed=500 + i, dtype=dtype, klm="chunkmean" if i % 2 else "iid",
                             with_dO=True)
    t = to_inputs(x)
    O, idx, sel, w, lse = hils.sparse_attn_fwd(t["Q"], t["K"], t["V"], t["Klm"], k, save_for_backward=True)
    ref = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k)
    gi = idx.cpu().numpy()
    check_selection(gi, ref["idx"], x["Q"], x["Klm"], 64, k)
    want = oracle.fwd(x["Q"], x["K"], x["V"], x["Klm"], 64, k, idx=gi)
    bar = tol(dtype)
    assert_close(f32(O), want["O"], "O", *bar)
    assert_close(f32(w), want["w"], "w", 1e-5, 1e-5)
    grads = hils.sparse_attn_bwd(t["Q"], t["K"], t["V"], t["Klm"], dev(x["dO"]), idx, w, lse, k)
    rb = oracle.bwd(x["Q"], x["K"], x["V"], x["Klm"], x["dO"], gi, 64, k)
    for name, got in zip(("dQ", "dK", "dV", "dKlm"), grads):
        assert_close(f32(got), rb[name], name, *bar)
