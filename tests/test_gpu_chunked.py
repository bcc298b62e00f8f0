"""GPU parity of chunked prefill (each request's queries are only the last
positions of its keys; the index is re-run over the chunk's tiles) against
the fp64 oracle, through the C ABI.

Bar: as every other shape (selections bit-exact outside the band, outputs
<= 2e-3 fp32 / 2e-2 bf16 and fp8); a chunk that starts on a block boundary
reproduces the whole prompt's rows bit for bit."""
import numpy as np
import pytest

from harness import assert_parity, compare, log, make_inputs, run_gpu, to_device
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


CHUNKS = [
    Workload("chunk-aligned-bf16", (2048,), 8, 2, 128, 128, "bf16", attractors=4, q_lens=(512,)),
    Workload("chunk-unaligned-bf16", (2000,), 8, 2, 128, 128, "bf16", attractors=4,
             q_lens=(700,)),
    Workload("chunk-varlen-mixed", (1500, 900, 400), 8, 2, 128, 128, "bf16", attractors=4,
             q_lens=(300, 900, 1)),
    Workload("chunk-empty-request", (1000, 600), 8, 2, 128, 64, "bf16", q_lens=(0, 600)),
    Workload("chunk-paged-p64", (3000, 1000), 8, 2, 128, 128, "bf16", page_size=64,
             attractors=4, q_lens=(1000, 333)),
    Workload("chunk-fp8-g8", (2500,), 16, 2, 128, 128, "fp8", sigma_c=1.5, q_lens=(600,)),
    Workload("chunk-f32-b64", (513,), 4, 1, 128, 64, "f32", q_lens=(200,)),
    Workload("chunk-b64-g1", (1500,), 2, 2, 64, 64, "bf16", q_lens=(250,)),
]


@pytest.mark.parametrize("w", CHUNKS, ids=lambda w: w.name)
def test_chunk_matches_oracle(w):
    inp = make_inputs(w, 31)
    dev = to_device(inp)
    for corr in (True, False):
        g = run_gpu(w, inp, correction=corr, dev_tensors=dev)
        rep = compare(w, inp, g, correction=corr)
        log(f"[chunk] {w.name} corr={corr}: {rep}")
        assert_parity(w, rep)


def test_chunk_with_kv_splits_matches_oracle():
    w = Workload("chunk-dense-split", (3000,), 8, 2, 128, 128, "bf16", alpha=0.0, attractors=4,
                 q_lens=(1000,))
    inp = make_inputs(w, 32)
    g = run_gpu(w, inp, kv_splits=4)
    rep = compare(w, inp, g)
    log(f"[chunk] {w.name}: {rep}")
    assert_parity(w, rep)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_block_aligned_chunk_equals_whole_prompt_rows(dtype):
    # the chunk's tiles are the whole prompt's tiles I >= i0, row for row
    whole = Workload("whole", (1536, 700), 8, 2, 128, 128, dtype, attractors=4)
    chunk = whole.replace(q_lens=(512, 700 - 256))  # offsets 1024 and 256: block boundaries
    inp_w = make_inputs(whole, 33)
    g_w = run_gpu(whole, inp_w, kv_splits=1)
    inp_c = make_inputs(chunk, 33)
    if dtype == "fp8":  # same codes and scales as the whole prompt's
        import torch
        starts = np.concatenate([[0], np.cumsum(whole.seqlens)])
        inp_c.q = torch.cat([inp_w.q[starts[b] + L - Lq:starts[b] + L]
                             for b, (L, Lq) in enumerate(zip(whole.seqlens, chunk.q_lens))])
        inp_c.q_scale = inp_w.q_scale
    g_c = run_gpu(chunk, inp_c, kv_splits=1)
    qs = 0
    for b, (L, Lq) in enumerate(zip(whole.seqlens, chunk.q_lens)):
        s = int(sum(whole.seqlens[:b]))
        rows = slice(s + L - Lq, s + L)
        assert np.array_equal(g_c.out[qs:qs + Lq], g_w.out[rows], equal_nan=True)
        assert np.array_equal(g_c.lse[:, qs:qs + Lq], g_w.lse[:, rows], equal_nan=True)
        qs += Lq
    assert np.array_equal(g_c.kbar, g_w.kbar)
