"""The HIP path on the worked example of tests/golden/fusion_ties_6chunks.json, whose answer is a closed
form (tests/golden/make_golden.py): selection with a tie toward the lower chunk index, own-chunk score
from its landmark, fusion weights and fused output, for the prefill and for decode steps."""
import numpy as np
import pytest
import torch

import golden_cases
from gpu_util import dev, f32, say, tol

pytestmark = pytest.mark.gpu


def _expect(case):
    sel = np.array([-np.inf if s is None else s for s in case["sel"]], np.float64)
    return np.array(case["idx"]), sel, np.array(case["w"]), np.array(case["o01"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_golden_worked_example(hils, gpu, dtype):
    g = golden_cases.load("fusion_ties_6chunks.json")
    x = golden_cases.fusion_ties_prefill(g, dtype)
    C, k = g["C"], g["k"]
    O, idx, sel, w, lse = hils.sparse_attn_fwd(dev(x["Q"]), dev(x["K"]), dev(x["V"]), dev(x["Klm"]), k,
                                              save_for_backward=True)
    torch.cuda.synchronize()
    gi, gs, gw, go = (a.cpu().numpy()[0, 0] for a in (idx, sel, w, O.float()))
    bar = tol(dtype)[0]
    for case in g["per_query_chunk"]:
        e_idx, e_sel, e_w, e_o = _expect(case)
        rows = slice(case["c"] * C, (case["c"] + 1) * C)
        say(f"golden {dtype} query chunk {case['c']}: idx {e_idx.tolist()}")
        assert (gi[rows] == e_idx).all(), case["c"]
        assert np.array_equal(np.isinf(gs[rows]), np.broadcast_to(np.isinf(e_sel), (C, e_sel.size)))
        fin = ~np.isinf(e_sel)
        assert np.abs(gs[rows][:, fin] - e_sel[fin]).max() < 1e-6
        assert np.abs(gw[rows] - e_w).max() < 1e-6
        assert np.abs(go[rows, :2] - e_o).max() < bar
        assert np.abs(go[rows, 2:]).max() == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [5, 64, 64 * 3 + 17, 64 * 4, 64 * 6 - 1])
def test_decode_golden_worked_example(hils, gpu, dtype, n):
    g = golden_cases.load("fusion_ties_6chunks.json")
    x = golden_cases.fusion_ties_decode(g, n, dtype)
    C, k = g["C"], g["k"]
    t = {name: dev(a) for name, a in x.items()}
    o, idx, w = hils.decode_step(t["q"], t["k_new"], t["v_new"], t["Kc"], t["Vc"], t["Klm"], n, k)
    torch.cuda.synchronize()
    e_idx, _, e_w, e_o = _expect(g["per_query_chunk"][n // C])
    assert (idx.cpu().numpy()[0, 0] == e_idx).all()
    assert np.abs(w.cpu().numpy()[0, 0] - e_w).max() < 1e-6
    go = f32(o)[0, 0]
    assert np.abs(go[:2] - e_o).max() < tol(dtype)[0]
    assert np.abs(go[2:]).max() == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_golden_worked_example(hils, gpu, dtype):
    g = golden_cases.load("fusion_ties_6chunks.json")
    x = golden_cases.fusion_ties_prefill(g, dtype)
    Q, K, V, Klm = (dev(x[n]) for n in ("Q", "K", "V", "Klm"))
    dO = dev(golden_cases.fusion_ties_dO(g, dtype))
    O, idx, sel, w, lse = hils.sparse_attn_fwd(Q, K, V, Klm, g["k"], save_for_backward=True)
    dQ, dK, dV, dKlm = hils.sparse_attn_bwd(Q, K, V, Klm, dO, idx, w, lse, g["k"])
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == golden_cases.fusion_ties_idx(g)).all()
    b = g["backward"]
    bar = tol(dtype)[0]
    for name, got, want in (("dQ", dQ, b["dQ0"]), ("dV", dV, b["dV0"]), ("dKlm", dKlm, b["dKlm0"])):
        a = f32(got)[0, 0]
        err = np.abs(a[:, 0] - np.asarray(want)).max()
        say(f"golden {dtype} {name}: max_abs={err:.3e}")
        assert err < bar, name
        assert np.abs(a[:, 1:]).max() < bar, name
    assert np.abs(f32(dK)).max() < bar
