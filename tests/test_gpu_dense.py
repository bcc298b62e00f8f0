"""GPU parity of the dense causal path (bslp_dense_prefill_attn: every key
j <= i, no index stage) against the fp64 oracle, through the C ABI.

Bar: output max-abs <= 2e-3 (fp32) / 2e-2 (bf16, fp8) and LSE max-abs <= 1e-3
(fp32) / 2e-2 against the textbook dense attention (fp8: the oracle's FP8
arithmetic over every causal block); bit-identical to the sparse path with
every block selected and mean correction off."""
import numpy as np
import pytest

import oracle
from harness import RequestView, log, make_inputs, out_tol, run_gpu, to_device
from workloads import SWEEP_BF16_64K, Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


def run_dense(w: Workload, inp, dev_tensors=None):
    import torch

    import block_sparse_long_pooled_amd as bslp
    q, k, v, table = dev_tensors or to_device(inp)
    prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.seqlens,
                             softmax_scale=w.scale, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             v_scale=inp.v_scale, page_table=table, page_size=w.page_size)
    T = sum(w.seqlens)
    odt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = torch.full((T, w.hq, w.d), float("nan"), dtype=odt, device="cuda")
    lse = torch.full((w.hq, T), float("nan"), dtype=torch.float32, device="cuda")
    bslp.dense_prefill_attn(prob, q, k, v, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def lse_tol(dtype: str) -> float:
    return 1e-3 if dtype == "f32" else 2e-2


DENSE = [
    Workload("dense-bf16-g4-ragged", (1000,), 8, 2, 128, 128, "bf16", attractors=4, vertical=3),
    Workload("dense-bf16-d64-b64", (777,), 2, 2, 64, 64, "bf16"),
    Workload("dense-fp8-g8-ragged", (1300,), 16, 2, 128, 128, "fp8", sigma_c=1.5),
    Workload("dense-f32-g4", (513,), 4, 1, 128, 64, "f32"),
    Workload("dense-varlen-bf16", (130, 1, 640, 384), 8, 2, 128, 64, "bf16", attractors=4),
    Workload("dense-paged-p16-fp8", (700, 260), 8, 2, 64, 64, "fp8", page_size=16),
]


@pytest.mark.parametrize("w", DENSE, ids=lambda w: w.name)
def test_dense_matches_textbook(w):
    log(f"[dense] {w.name}")
    inp = make_inputs(w, 4)
    out, lse = run_dense(w, inp)
    start = 0
    err_o = err_l = 0.0
    for b, L in enumerate(w.seqlens):
        rv = RequestView(w, inp, b)
        if w.dtype == "fp8":
            # the pages' FP8 arithmetic over every causal block, tile by tile
            for h in range(w.hkv):
                k_h, v_h, kbar_h, vbar_h = rv.head(h)
                for I in range(-(-L // w.block)):
                    pos, heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I)
                    O, l = oracle.attend_rows_fp8(pos, rows, k_h, v_h, list(range(I + 1)), [],
                                                  w.block, w.scale, rv.ks, rv.vs)
                    err_o = max(err_o, float(np.abs(out[start + pos, heads] - O).max()))
                    err_l = max(err_l, float(np.abs(lse[heads, start + pos] - l).max()))
            start += L
            continue
        k = np.stack([rv.head(h)[0] for h in range(w.hkv)], axis=1)
        v = np.stack([rv.head(h)[1] for h in range(w.hkv)], axis=1)
        Od, lsed = oracle.dense_causal_reference(rv.q, k, v, w.scale)
        err_o = max(err_o, float(np.abs(out[start:start + L] - Od).max()))
        err_l = max(err_l, float(np.abs(lse[:, start:start + L] - lsed).max()))
        start += L
    log(f"[dense] {w.name}: out_maxabs={err_o:.3e} lse_maxabs={err_l:.3e}")
    assert err_o <= out_tol(w.dtype)
    assert err_l <= lse_tol(w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_dense_equals_sparse_all_selected_bitwise(dtype):
    # alpha = 0 keeps every causal block; without correction the sparse path
    # walks exactly the dense path's blocks in the same order
    w = Workload("dense-vs-sparse", (1000, 300), 8, 2, 128, 128, dtype, attractors=4)
    inp = make_inputs(w, 6)
    dev = to_device(inp)
    g = run_gpu(w, inp, alpha=0.0, correction=False, dev_tensors=dev)
    out, lse = run_dense(w, inp, dev_tensors=dev)
    assert np.array_equal(out, g.out, equal_nan=True)
    assert np.array_equal(lse, g.lse, equal_nan=True)


def test_dense_64k_sampled_rows():
    w = SWEEP_BF16_64K
    inp = make_inputs(w, 0)
    out, lse = run_dense(w, inp)
    rv = RequestView(w, inp, 0)
    N = -(-w.seqlens[0] // w.block)
    rng = np.random.default_rng(0)
    err_o = err_l = 0.0
    for h in (0, w.hkv - 1):
        k_h, v_h, kbar_h, vbar_h = rv.head(h)
        for I in sorted({0, 1, N // 2, N - 1, *rng.integers(0, N, 2).tolist()}):
            pos, heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I)
            pick = rng.choice(len(pos), size=min(24, len(pos)), replace=False)
            O, l = oracle.attend_rows(pos[pick], rows[pick], k_h, v_h, kbar_h, vbar_h,
                                      list(range(I + 1)), [], w.block, w.scale)
            err_o = max(err_o, float(np.abs(out[pos[pick], heads[pick]] - O).max()))
            err_l = max(err_l, float(np.abs(lse[heads[pick], pos[pick]] - l).max()))
    log(f"[dense] {w.name} sampled: out_maxabs={err_o:.3e} lse_maxabs={err_l:.3e}")
    assert err_o <= out_tol(w.dtype)
    assert err_l <= lse_tol(w.dtype)
