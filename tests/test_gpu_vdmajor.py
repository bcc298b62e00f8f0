"""fp8 inputs with V in the d-major layout ([Hkv, d, kv tokens], or [pages,
Hkv, d, page] when paged; the V-layout bullet of the "FlashPrefill V2" FP8
paragraph): every output equals the row-major run's bitwise, the pooled
values to float32 rounding, including paged V whose bytes past each request
hold the e4m3 NaN code.  The row-major fp8 path itself is compared with the
oracle in test_gpu_parity.py; one d-major case is compared here too."""
import numpy as np
import pytest

from harness import (assert_parity, compare, log, make_inputs, run_gpu, to_device, v_dmajor)
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


CASES = [
    (Workload("vd-varlen-d128-b64", (700, 1300, 129), 8, 2, 128, 64, "fp8"), {}),
    (Workload("vd-d64-b128-g4", (1000,), 16, 4, 64, 128, "fp8"), {}),
    (Workload("vd-no-correction", (1500,), 8, 2, 128, 64, "fp8", correction=False), {}),
    (Workload("vd-split3", (3000,), 8, 2, 128, 64, "fp8"), {"kv_splits": 3}),
    (Workload("vd-chunk", (2048, 900), 8, 2, 128, 64, "fp8", q_lens=(700, 900)), {}),
    (Workload("vd-paged-64", (900, 333), 8, 2, 128, 64, "fp8", page_size=64), {}),
    (Workload("vd-paged-128-b128", (1025,), 8, 2, 128, 128, "fp8", page_size=128), {}),
]


def _same(a, b, name):
    assert np.array_equal(a, b, equal_nan=True), name


@pytest.mark.parametrize("w,kw", CASES, ids=[c[0].name for c in CASES])
def test_dmajor_v_equals_row_major(w, kw):
    inp = make_inputs(w, 3)
    q, k, v, table = to_device(inp)
    log(f"[vdmajor] {w.name} {kw}")
    g_rows = run_gpu(w, inp, dev_tensors=(q, k, v, table), **kw)
    g_dm = run_gpu(w, inp, dev_tensors=(q, k, v_dmajor(w, v), table), v_dmajor=True, **kw)
    for name in ("kbar", "scores", "counts", "cu", "idx", "out", "lse"):
        _same(getattr(g_rows, name), getattr(g_dm, name), name)
    np.testing.assert_allclose(g_dm.vbar, g_rows.vbar, rtol=1e-6, atol=0)


def test_dmajor_v_ignores_bytes_past_each_request():
    # paged d-major V whose unused page slots hold 0x7f, the e4m3 NaN code
    import torch
    w = Workload("vd-paged-nan", (900, 333, 70), 8, 2, 128, 64, "fp8", page_size=64)
    inp = make_inputs(w, 5)
    q, k, v, table = to_device(inp)
    g_rows = run_gpu(w, inp, dev_tensors=(q, k, v, table))
    vd = v_dmajor(w, v)  # [pages, Hkv, d, page]
    used = torch.zeros(vd.shape[0], vd.shape[3], dtype=torch.bool, device=vd.device)
    t = inp.table
    for b, L in enumerate(w.seqlens):
        for j in range(L):
            used[int(t[b, j // 64]), j % 64] = True
    vd = torch.where(used[:, None, None, :], vd, torch.full_like(vd, 0x7F))
    g_dm = run_gpu(w, inp, dev_tensors=(q, k, vd, table), v_dmajor=True)
    for name in ("out", "lse", "idx", "kbar", "scores"):
        _same(getattr(g_rows, name), getattr(g_dm, name), name)
    np.testing.assert_allclose(g_dm.vbar, g_rows.vbar, rtol=1e-6, atol=0)


def test_dmajor_v_dense_equals_row_major():
    import torch

    import block_sparse_long_pooled_amd as bslp
    w = Workload("vd-dense", (1100, 400), 8, 2, 128, 64, "fp8")
    inp = make_inputs(w, 2)
    q, k, v, _ = to_device(inp)
    res = []
    for dm, vv in ((False, v), (True, v_dmajor(w, v))):
        prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.seqlens, softmax_scale=w.scale,
                                 q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale,
                                 v_dmajor=dm)
        out = torch.full((q.shape[0], w.hq, w.d), float("nan"), dtype=torch.bfloat16, device=q.device)
        lse = torch.full((w.hq, q.shape[0]), float("nan"), dtype=torch.float32, device=q.device)
        bslp.dense_prefill_attn(prob, q, k, vv, out, lse)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), lse.cpu().numpy()))
    _same(res[0][0], res[1][0], "out")
    _same(res[0][1], res[1][1], "lse")
    assert np.isfinite(res[1][0]).all()


def test_dmajor_v_oracle_parity():
    w = Workload("vd-oracle", (1200, 500), 8, 2, 128, 64, "fp8")
    inp = make_inputs(w, 7)
    q, k, v, table = to_device(inp)
    g = run_gpu(w, inp, dev_tensors=(q, k, v_dmajor(w, v), table), v_dmajor=True)
    rep = compare(w, inp, g)
    log(f"[vdmajor] {w.name}: {rep}")
    assert_parity(w, rep)
