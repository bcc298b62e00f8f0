"""The attention entry point that allocates nothing, through the C ABI: its
outputs equal those of bslp_sparse_prefill_attn (same kernels, same work
split) on two calls in a row, the second on a smaller problem, so results
left in the shared device scratch by the first call cannot leak into the
second.  Host-side limits are checked without a GPU in test_abi.py."""
import numpy as np
import pytest

from harness import log, make_inputs, to_device
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


def _both(w, seed, kv_splits=0):
    import torch

    import block_sparse_long_pooled_amd as bslp
    inp = make_inputs(w, seed)
    q, k, v, table = to_device(inp)
    prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.query_lens,
                             softmax_scale=w.scale, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             v_scale=inp.v_scale, page_table=table, page_size=w.page_size,
                             kv_splits=kv_splits)
    params = bslp.make_params(w.alpha, w.sink, w.window, w.recent, w.correction)
    bufs = bslp.Buffers(prob)
    bslp.block_scores(prob, q, k, v, bufs.kbar, bufs.vbar, bufs.scores)
    bslp.select_blocks(prob, params, q, bufs.kbar, bufs.scores, bufs.counts, bufs.cu, bufs.idx)
    bslp.sparse_prefill_attn(prob, params, q, k, v, bufs.kbar, bufs.vbar, bufs.cu, bufs.idx,
                             bufs.out, bufs.lse, bufs.workspace)
    out2 = torch.full_like(bufs.out, float("nan"))
    lse2 = torch.full_like(bufs.lse, float("nan"))
    bslp.sparse_prefill_attn_noalloc(prob, params, q, k, v, bufs.kbar, bufs.vbar, bufs.cu,
                                     bufs.idx, out2, lse2)
    torch.cuda.synchronize()
    a, b = bufs.out.float().cpu().numpy(), out2.float().cpu().numpy()
    la, lb = bufs.lse.cpu().numpy(), lse2.cpu().numpy()
    assert np.isfinite(b).all() and not np.isnan(lb).any()
    err = float(np.abs(a - b).max())
    log(f"[noalloc] {w.name} splits={kv_splits}: out max-abs vs workspace call {err:.3e}")
    assert err <= (2e-3 if w.dtype == "f32" else 2e-2)
    # the same kernels on the same work: bit for bit
    assert np.array_equal(a, b) and np.array_equal(la, lb)


@pytest.mark.parametrize("kv_splits", [0, 3])
def test_noalloc_matches_workspace_call_twice(kv_splits):
    # with 3 forced splits the partial results (3 x T x Hq x (d + 2) floats)
    # must fit the 32 MiB scratch: 21 MB for the first problem
    big = Workload("noalloc-big-bf16", (3000, 1200) if kv_splits == 0 else (1200, 500),
                   16 if kv_splits == 0 else 8, 4 if kv_splits == 0 else 2, 128, 128, "bf16",
                   attractors=4)
    small = Workload("noalloc-small-fp8", (700,), 8, 2, 64, 64, "fp8", sigma_c=1.5)
    _both(big, 1, kv_splits)
    _both(small, 2, kv_splits)


def test_noalloc_f32_and_paged():
    _both(Workload("noalloc-f32", (513,), 4, 1, 128, 64, "f32"), 3)
    _both(Workload("noalloc-paged", (900, 400), 8, 2, 128, 128, "bf16", page_size=64,
                   attractors=4), 4)
