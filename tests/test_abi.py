"""The C ABI library loads, exports what include/hils.h declares, and rejects bad arguments on the host.

Runs without a GPU: every call below fails validation before any HIP call is made.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hils.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)  # aligned non-null address; never dereferenced by a failing call
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(hils_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib(hils):
    return hils._lib


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("hils_landmark_scores", "hils_topk_select", "hils_sparse_attn_fwd", "hils_decode_step",
              "hils_sparse_attn_bwd", "hils_workspace_size", "hils_last_error", "hils_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in include/hils.h but not exported"


def test_version_and_error_string(lib, hils):
    assert hils.version() >= 10000
    assert isinstance(lib.hils_last_error(), bytes)


def _topk(lib, Q=FAKE, Klm=FAKE, idx=FAKE, sel=FAKE, w=None, B=1, H=1, L=128, d=64, C=64, k=4, scale=0.125, dt=0):
    return lib.hils_topk_select(Q, Klm, idx, sel, w, B, H, L, d, C, k, scale, dt, None, 0, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Q=None), INVALID, "Q must not be null"),
    (dict(idx=None), INVALID, "idx must not be null"),
    (dict(Klm=MISALIGNED), INVALID, "aligned"),
    (dict(w=MISALIGNED), INVALID, "aligned"),
    (dict(d=96), UNSUPPORTED, "head dim"),
    (dict(C=32), UNSUPPORTED, "chunk size"),
    (dict(L=100), INVALID, "multiple of C"),
    (dict(L=0), INVALID, "L must be"),
    (dict(B=0), INVALID, "B and H"),
    (dict(k=0), UNSUPPORTED, "top-k"),
    (dict(k=17), UNSUPPORTED, "top-k"),
    (dict(dt=7), INVALID, "element type"),
    (dict(scale=0.0), INVALID, "scale"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(L=64 * 20000), UNSUPPORTED, "chunks"),
])
def test_topk_validation(lib, kw, status, msg):
    assert _topk(lib, **kw) == status
    assert msg in lib.hils_last_error().decode()


def test_topk_workspace_checks(lib, hils):
    need = hils.workspace_size(hils.OP_TOPK, 1, 1, 128, 64, 64, 4)
    args = [FAKE] * 4 + [None, 1, 1, 128, 64, 64, 4, 0.125, 0]
    assert lib.hils_topk_select(*args, None, need, None) == WORKSPACE
    assert lib.hils_topk_select(*args, FAKE, need - 16, None) == WORKSPACE
    assert "too small" in lib.hils_last_error().decode()


def test_fwd_workspace_checks(lib, hils):
    need = hils.workspace_size(hils.OP_FWD, 1, 2, 1024, 64, 64, 4)
    assert need > 0
    args = [FAKE] * 6 + [1, FAKE, None, None, 1, 2, 1024, 64, 64, 4, 0.125, 0]
    assert lib.hils_sparse_attn_fwd(*args, None, need, None) == WORKSPACE
    assert lib.hils_sparse_attn_fwd(*args, FAKE, need - 1, None) == WORKSPACE
    assert "too small" in lib.hils_last_error().decode()
    bad_select = [FAKE] * 6 + [2, FAKE, None, None, 1, 2, 1024, 64, 64, 4, 0.125, 0]
    assert lib.hils_sparse_attn_fwd(*bad_select, FAKE, need, None) == INVALID


def test_workspace_size_grows_with_problem(hils):
    a = hils.workspace_size(hils.OP_FWD, 1, 1, 1024, 64, 64, 4)
    b = hils.workspace_size(hils.OP_FWD, 1, 2, 1024, 64, 64, 4)
    c = hils.workspace_size(hils.OP_FWD, 1, 1, 2048, 128, 64, 8)
    assert 0 < a < b and a < c
    # the selection keeps a copy of the landmarks, rows padded to a multiple of 64
    assert hils.workspace_size(hils.OP_TOPK, 1, 1, 1024, 64, 64, 4) == 64 * 64 * 2
    assert hils.workspace_size(hils.OP_TOPK, 2, 3, 64 * 65, 128, 64, 4) == 6 * 128 * 128 * 2
    with pytest.raises(hils.HilsError):
        hils.workspace_size(hils.OP_FWD, 1, 1, 1000, 64, 64, 4)


def test_scores_validation(lib):
    assert lib.hils_landmark_scores(FAKE, FAKE, None, 1, 1, 128, 64, 64, 0.125, 0, None) == INVALID
    assert lib.hils_landmark_scores(FAKE, FAKE, FAKE, 1, 1, 128, 80, 64, 0.125, 0, None) == UNSUPPORTED


def test_retrieval_query_entry_points_validate(lib, hils):
    need = hils.workspace_size(hils.OP_FWD, 1, 2, 1024, 64, 64, 4)
    tail = [1, FAKE, None, None, 1, 2, 1024, 64, 64, 4, 0.125, 0]
    # a misaligned retrieval query is rejected; a null one is the plain entry point's workspace check
    assert lib.hils_sparse_attn_fwd_rq(FAKE, MISALIGNED, *([FAKE] * 5), *tail, FAKE, need, None) == INVALID
    assert "Q_ret" in lib.hils_last_error().decode()
    assert lib.hils_sparse_attn_fwd_rq(FAKE, None, *([FAKE] * 5), *tail, None, need, None) == WORKSPACE
    # backward: Q_ret and dQ_ret come together
    nb = hils.workspace_size(hils.OP_BWD, 1, 2, 1024, 64, 64, 4)
    dims = [1, 2, 1024, 64, 64, 4, 0.125, 0]
    assert lib.hils_sparse_attn_bwd_rq(FAKE, FAKE, *([FAKE] * 8), None, *([FAKE] * 3), *dims, FAKE, nb,
                                       None) == INVALID
    assert "together" in lib.hils_last_error().decode()
    assert lib.hils_sparse_attn_bwd_rq(FAKE, None, *([FAKE] * 8), FAKE, *([FAKE] * 3), *dims, FAKE, nb,
                                       None) == INVALID
    # decode: misaligned q_ret
    nd = hils.workspace_size(hils.OP_DECODE, 1, 2, 1024, 64, 64, 4)
    assert lib.hils_decode_step_rq(FAKE, MISALIGNED, *([FAKE] * 5), 100, 1024, FAKE, FAKE, FAKE, 1, 2, 64, 64, 4,
                                   0.125, 0, FAKE, nd, None) == INVALID
    assert "q_ret" in lib.hils_last_error().decode()


def test_landmark_free_entry_points_validate(lib, hils):
    # chunk means: more chunks than the keys hold, or than K_lm has rows
    assert lib.hils_chunk_means(FAKE, FAKE, 1, 2, 640, 10, 11, 64, 64, 0, None) == INVALID
    assert lib.hils_chunk_means(FAKE, FAKE, 1, 2, 1024, 8, 9, 64, 64, 0, None) == INVALID
    assert "n_chunks" in lib.hils_last_error().decode()
    assert lib.hils_chunk_means(FAKE, FAKE, 1, 2, 640, 10, 10, 96, 64, 0, None) == UNSUPPORTED
    assert lib.hils_chunk_means(FAKE, None, 1, 2, 640, 10, 10, 64, 64, 0, None) == INVALID
    # forward: the landmark output is required
    need = hils.workspace_size(hils.OP_FWD, 1, 2, 1024, 64, 64, 4)
    tail = [1, FAKE, None, None, 1, 2, 1024, 64, 64, 4, 0.125, 0]
    assert lib.hils_sparse_attn_fwd_lf(FAKE, None, FAKE, FAKE, None, FAKE, FAKE, *tail, FAKE, need, None) == INVALID
    assert lib.hils_sparse_attn_fwd_lf(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, *tail, None, need, None) == WORKSPACE
    nd = hils.workspace_size(hils.OP_DECODE, 1, 2, 1024, 64, 64, 4)
    assert lib.hils_decode_step_lf(FAKE, None, *([FAKE] * 5), 1024, 1024, FAKE, FAKE, FAKE, 1, 2, 64, 64, 4,
                                   0.125, 0, FAKE, nd, None) == INVALID
    assert "n_ctx" in lib.hils_last_error().decode()


def test_landmark_free_backward_validates(lib, hils):
    nb = hils.workspace_size(hils.OP_BWD, 1, 2, 1024, 64, 64, 4)
    dims = [1, 2, 1024, 64, 64, 4, 0.125, 0]
    # Q_ret without dQ_ret; fp32 at d = 128 is accepted, and a workspace sized for d = 64 is then too small
    assert lib.hils_sparse_attn_bwd_lf(FAKE, FAKE, *([FAKE] * 8), None, *([FAKE] * 3), *dims, FAKE, nb,
                                       None) == INVALID
    assert lib.hils_sparse_attn_bwd_lf(FAKE, None, *([FAKE] * 8), None, *([FAKE] * 3), 1, 2, 1024, 128, 64, 4,
                                       0.125, 1, FAKE, nb, None) == WORKSPACE


def test_paged_decode_validates(lib, hils):
    nd = hils.workspace_size(hils.OP_DECODE, 2, 2, 64 * 10, 64, 64, 4)
    head = [FAKE] * 7 + [1, FAKE]  # ..., K_lm_pages, m = 1 landmark per chunk, page_table
    # n_ctx_max beyond the table, a zero-page pool, and a bad landmark_free flag
    assert lib.hils_decode_step_paged(*head, 5, 10, FAKE, 640, 0, FAKE, FAKE, FAKE, 2, 2, 64, 64, 4, 0.125, 0,
                                      FAKE, nd, None) == INVALID
    assert "n_ctx_max" in lib.hils_last_error().decode()
    assert lib.hils_decode_step_paged(*head, 0, 10, FAKE, 100, 0, FAKE, FAKE, FAKE, 2, 2, 64, 64, 4, 0.125, 0,
                                      FAKE, nd, None) == INVALID
    assert lib.hils_decode_step_paged(*head, 5, 10, FAKE, 100, 2, FAKE, FAKE, FAKE, 2, 2, 64, 64, 4, 0.125, 0,
                                      FAKE, nd, None) == INVALID
    assert lib.hils_decode_step_paged(*head, 5, 10, FAKE, 100, 0, FAKE, FAKE, FAKE, 2, 2, 64, 64, 4, 0.125, 0,
                                      FAKE, nd - 16, None) == WORKSPACE
    # landmarks per chunk: 1..16, and one only with landmark-free chunks
    for m, lf, status in ((0, 0, UNSUPPORTED), (17, 0, UNSUPPORTED), (2, 1, INVALID)):
        assert lib.hils_decode_step_paged(*([FAKE] * 7), m, FAKE, 5, 10, FAKE, 100, lf, FAKE, FAKE, FAKE, 2, 2, 64,
                                          64, 4, 0.125, 0, FAKE, nd, None) == status
        assert "landmark" in lib.hils_last_error().decode()


def test_multi_landmark_forward_validates(lib, hils):
    need = hils.workspace_size(hils.OP_FWD_ML, 1, 2, 1024, 64, 64, 4)
    # the plain forward's workspace: no chunk score matrix is formed
    assert need == hils.workspace_size(hils.OP_FWD, 1, 2, 1024, 64, 64, 4) > 0
    tail = [1, FAKE, None, None, 1, 2, 1024, 64, 64, 4, 0.125, 0]
    assert lib.hils_sparse_attn_fwd_ml(FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, FAKE, *tail, FAKE, need,
                                       None) == UNSUPPORTED
    assert lib.hils_sparse_attn_fwd_ml(FAKE, None, FAKE, FAKE, FAKE, 17, FAKE, FAKE, *tail, FAKE, need,
                                       None) == UNSUPPORTED
    assert lib.hils_sparse_attn_fwd_ml(FAKE, None, FAKE, FAKE, FAKE, 2, FAKE, FAKE, *tail, FAKE, need - 16,
                                       None) == WORKSPACE


def test_multi_landmark_decode_validates(lib, hils):
    nd = hils.workspace_size(hils.OP_DECODE, 1, 2, 1024, 64, 64, 4)
    for m in (0, 17):
        assert lib.hils_decode_step_ml(FAKE, None, *([FAKE] * 5), m, 100, 1024, FAKE, FAKE, FAKE, 1, 2, 64, 64, 4,
                                       0.125, 0, FAKE, nd, None) == UNSUPPORTED


def test_noalloc_decode_validation(lib):
    """The no-allocation decode step rejects, before any HIP call, batches whose scratch exceeds the fixed
    array and the argument errors of the workspace step."""
    args = [FAKE] * 6 + [100, 1024] + [FAKE] * 3
    assert lib.hils_decode_step_noalloc(*args, 1, 700, 128, 64, 8, ctypes.c_float(0.125), 0, None) == UNSUPPORTED
    assert "scratch" in lib.hils_last_error().decode()
    assert lib.hils_decode_step_noalloc(*args, 1, 2, 96, 64, 8, ctypes.c_float(0.125), 0, None) == UNSUPPORTED
    assert lib.hils_decode_step_noalloc(*[FAKE] * 6, 2000, 1024, *[FAKE] * 3, 1, 2, 64, 64, 8,
                                        ctypes.c_float(0.125), 0, None) == INVALID
    assert "n_ctx" in lib.hils_last_error().decode()
    assert lib.hils_decode_step_noalloc(*[FAKE] * 5, None, 100, 1024, *[FAKE] * 3, 1, 2, 64, 64, 8,
                                        ctypes.c_float(0.125), 0, None) == INVALID


def test_routing_pair_index_division_is_exact():
    """The routing kernels split a lane's pair number f into (query f // k, slot f % k) with one float
    product, truncating (f + 1/2) * fl(1/k) in fp32; that must equal the integer quotient for every pair
    number a routing run can hold (below 1024 queries x 16 slots, checked here up to 2^15) and every k
    up to 32."""
    import numpy as np

    f = np.arange(1 << 15, dtype=np.int64)
    for k in range(1, 33):
        rk = np.float32(1.0) / np.float32(k)
        q = ((f.astype(np.float32) + np.float32(0.5)) * rk).astype(np.int64)
        np.testing.assert_array_equal(q, f // k, err_msg=f"k={k}")
