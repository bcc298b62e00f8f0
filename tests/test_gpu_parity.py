"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bar: selected-block lists bit-exact outside the 1e-5 threshold band; output
max-abs <= 2e-3 (fp32) / 2e-2 (bf16, fp8) against the oracle evaluated on
the validated selection; pooled means and scores to float32 accuracy."""
import numpy as np
import pytest

from harness import (assert_parity, compare, log, make_inputs, run_gpu, sample_tiles,
                     segments, to_device)
from workloads import (CHUNK_BF16_64K, FP8_128K, GQA_BF16_16K, PAGED_VARLEN, SWEEP_ALPHAS,
                       SWEEP_BF16_64K, TINY_F32, Workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


def _full(w, seed, **kw):
    log(f"[parity] {w.name} seed={seed} {kw}")
    inp = make_inputs(w, seed)
    g = run_gpu(w, inp, **kw)
    rep = compare(w, inp, g, **kw)
    log(f"[parity] {w.name} seed={seed}: {rep} gpu_ms={g.ms:.1f}")
    assert_parity(w, rep)
    return inp, g, rep


# ----------------------------------------------------------------- tiny fp32

@pytest.mark.parametrize("seed", TINY_F32.seeds)
def test_tiny_f32_all_seeds(seed):
    _full(TINY_F32, seed)


# ----------------------------------------------------------------- small shapes, ragged tails

SMALL = [
    Workload("bf16-ragged-g4", (1000,), 8, 2, 128, 128, "bf16", attractors=4, vertical=3),
    Workload("bf16-d64-b64-g1", (777,), 2, 2, 64, 64, "bf16"),
    Workload("fp8-g8-ragged", (1300,), 16, 2, 128, 128, "fp8", sigma_c=1.5),
    Workload("f32-g4-d128", (513,), 4, 1, 128, 64, "f32"),
    Workload("varlen-bf16", (130, 1, 640, 384), 8, 2, 128, 64, "bf16", attractors=4),
    Workload("paged-varlen-bf16", (300, 1024, 77), 8, 4, 128, 128, "bf16", page_size=64,
             attractors=4, vertical=4),
    Workload("paged-p16-fp8", (700, 260), 8, 2, 64, 64, "fp8", page_size=16),
    Workload("no-forced-blocks", (1024,), 4, 1, 64, 64, "bf16", sink=0, window=0, recent=0,
             alpha=0.3),
    Workload("wide-forced", (1536,), 4, 2, 128, 64, "bf16", sink=3, window=4, recent=2,
             alpha=0.5),
    # more KV heads than one pooling workgroup covers (16 at d = 128, 32 at
    # d = 64): head groups of 16 + 4 and 32 + 8
    Workload("kv-heads-20-d128", (600,), 20, 20, 128, 64, "bf16", attractors=4),
    Workload("kv-heads-40-d64-fp8", (333,), 40, 40, 64, 64, "fp8", sigma_c=1.5),
    # 17 heads of 64 dims: 136 threads per token row, one row group
    Workload("kv-heads-17-d64-f32", (200,), 17, 17, 64, 64, "f32"),
    # 129 blocks: tiles I = 0..128 cover one, two and three correction chunks
    # of 64 pooled blocks, the last with a single block
    Workload("corr-chunks-129-blocks", (8200,), 4, 1, 64, 64, "bf16", attractors=4),
    Workload("corr-chunks-fp8", (8200,), 8, 1, 64, 64, "fp8", sigma_c=1.5),
    # group size 16: 2048-row tiles at B = 128 (block scores beyond the
    # matrix-core kernel's 1024 rows), 1024-row tiles at B = 64 (16 waves)
    Workload("g16-b128-bf16", (1000,), 32, 2, 128, 128, "bf16", attractors=4),
    Workload("g16-b128-fp8", (700,), 16, 1, 64, 128, "fp8", sigma_c=1.5),
    Workload("g16-b64-bf16", (900,), 16, 1, 128, 64, "bf16", attractors=4),
    Workload("g16-b64-fp8", (777,), 32, 2, 128, 64, "fp8", sigma_c=1.5),
    # group sizes that are not powers of two: packed-row divmod, partial
    # row blocks and row tiles
    Workload("g3-hq12-hkv4-bf16", (1100,), 12, 4, 128, 128, "bf16", attractors=4),
    Workload("g3-hq12-hkv4-fp8", (650,), 12, 4, 128, 64, "fp8", sigma_c=1.5),
    Workload("g5-hq10-hkv2-bf16", (900,), 10, 2, 64, 64, "bf16"),
    Workload("g6-hq12-hkv2-bf16", (1300,), 12, 2, 128, 128, "bf16", attractors=4, vertical=3),
    Workload("g12-hq24-hkv2-fp8", (500,), 24, 2, 128, 128, "fp8", sigma_c=1.5),
    Workload("g7-hq7-hkv1-f32", (300,), 7, 1, 64, 64, "f32"),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_shapes(w):
    _full(w, 3)


# ----------------------------------------------------------------- chunks with nothing to mask

# No sink block and a high threshold: tiles past block 64 leave whole
# correction chunks of 64 pooled blocks with none selected, which the
# kernels run without the masking pass ("FlashPrefill V2", Sec. 3.2 / Fig. 3
# paragraph: the todo set is every valid block not selected).
UNSELECTED_CHUNKS = [
    Workload("corr-unselected-bf16", (8200,), 4, 1, 64, 64, "bf16", sink=0, window=1,
             recent=0, alpha=0.5),
    Workload("corr-unselected-fp8", (8200,), 8, 1, 64, 64, "fp8", sigma_c=1.5, sink=0,
             window=1, recent=0, alpha=0.5),
]


@pytest.mark.parametrize("w", UNSELECTED_CHUNKS, ids=lambda w: w.name)
def test_correction_chunks_with_nothing_to_mask(w):
    _, g, _ = _full(w, 3)
    # (tile, chunk) pairs whose chunk holds 64 valid blocks (J <= I - 1), none
    # selected: the case must occur for the test to cover it
    full_unselected = 0
    for (_, _, I, s, _) in segments(w.seqlens, w.hkv, w.block):
        sel = np.zeros(I + 1, dtype=bool)
        sel[g.idx[g.cu[s]:g.cu[s + 1]]] = True
        for c in range(I // 64):
            full_unselected += not sel[64 * c:64 * c + 64].any()
    log(f"[parity] {w.name}: {full_unselected} full correction chunks with no selected block")
    assert full_unselected > 0


@pytest.mark.parametrize("correction", [True, False])
def test_alpha_zero_is_dense(correction):
    w = Workload("dense-bf16", (700,), 8, 2, 128, 64, "bf16", alpha=0.0, sink=0, window=0,
                 recent=0, correction=correction)
    inp, g, rep = _full(w, 5)
    assert rep.selected == rep.blocks  # every causal block kept
    # and against the textbook dense attention
    import oracle
    from harness import RequestView
    rv = RequestView(w, inp, 0)
    k = np.stack([rv.head(h)[0] for h in range(w.hkv)], axis=1)
    v = np.stack([rv.head(h)[1] for h in range(w.hkv)], axis=1)
    Od, lsed = oracle.dense_causal_reference(rv.q, k, v, w.scale)
    assert np.abs(g.out - Od).max() < 2e-2
    assert np.abs(g.lse - lsed).max() < 2e-2


# ----------------------------------------------------------------- 16K GQA bf16, full compare

@pytest.mark.parametrize("seed", GQA_BF16_16K.seeds)
def test_gqa_bf16_16k_full(seed):
    _full(GQA_BF16_16K, seed)


# ----------------------------------------------------------------- equivalences

def test_paged_equals_contiguous_bitwise():
    w = Workload("pg", (900, 2048, 128), 8, 2, 128, 128, "bf16", page_size=128, attractors=4)
    inp = make_inputs(w, 1)
    g_paged = run_gpu(w, inp)
    inp_c = make_inputs(w.replace(page_size=0), 1)
    g_cont = run_gpu(w.replace(page_size=0), inp_c)
    for name in ("kbar", "vbar", "scores", "counts", "cu", "idx", "out", "lse"):
        a, b = getattr(g_paged, name), getattr(g_cont, name)
        assert np.array_equal(a, b, equal_nan=True), name


@pytest.mark.parametrize("kv_splits", [1, 3])
def test_varlen_equals_standalone_bitwise(kv_splits):
    # with a fixed split count every request's work is cut the same way
    # whatever it is packed with (the automatic count depends on the batch)
    lens = (640, 1000, 256)
    w = Workload("vl", lens, 8, 2, 128, 64, "bf16", attractors=4)
    inp = make_inputs(w, 2)
    g = run_gpu(w, inp, kv_splits=kv_splits)
    starts = np.concatenate([[0], np.cumsum(lens)])
    for b, L in enumerate(lens):
        wb = w.replace(seqlens=(L,))
        sl = slice(int(starts[b]), int(starts[b + 1]))
        inp_b = make_inputs(w, 2)  # same draws; take request b's rows
        inp_b.q, inp_b.k, inp_b.v = (t[sl].contiguous() for t in (inp.q, inp.k, inp.v))
        gb = run_gpu(wb, inp_b, kv_splits=kv_splits)
        assert np.array_equal(gb.out, g.out[sl], equal_nan=True)
        assert np.array_equal(gb.lse, g.lse[:, sl], equal_nan=True)


def test_pool_and_score_halves_equal_block_scores():
    # bslp_pool_kv + bslp_score_blocks enqueue exactly bslp_block_scores' work
    import torch

    import block_sparse_long_pooled_amd as bslp
    for w in (Workload("halves-bf16", (900, 300), 8, 2, 128, 128, "bf16", attractors=4),
              Workload("halves-fp8-paged", (700,), 8, 2, 64, 64, "fp8", page_size=16)):
        inp = make_inputs(w, 4)
        q, k, v, table = to_device(inp)
        prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.seqlens,
                                 q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale,
                                 page_table=table, page_size=w.page_size)
        a, b = bslp.Buffers(prob), bslp.Buffers(prob)
        bslp.block_scores(prob, q, k, v, a.kbar, a.vbar, a.scores)
        bslp.pool_kv(prob, k, v, b.kbar, b.vbar)
        bslp.score_blocks(prob, q, b.kbar, b.scores)
        torch.cuda.synchronize()
        for n in ("kbar", "vbar", "scores"):
            assert torch.equal(getattr(a, n), getattr(b, n)), (w.name, n)


def test_select_leaves_scores_bitwise_unchanged():
    # the selection's count pass negates the scores of the uncertain blocks it
    # drops after the exact re-decision, and the emit pass restores them; the
    # 64K workload has hundreds of segments with a score in the uncertain
    # band (2e-3 relative around alpha times the row maximum), so the path runs
    import torch

    import block_sparse_long_pooled_amd as bslp
    w = SWEEP_BF16_64K
    inp = make_inputs(w, 0)
    q, k, v, _ = to_device(inp)
    prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.seqlens, softmax_scale=w.scale)
    params = bslp.make_params(w.alpha, w.sink, w.window, w.recent, w.correction)
    bufs = bslp.Buffers(prob)
    bslp.pool_kv(prob, k, v, bufs.kbar, bufs.vbar)
    bslp.score_blocks(prob, q, bufs.kbar, bufs.scores)
    before = bufs.scores.clone()
    for _ in range(2):
        bslp.select_blocks(prob, params, q, bufs.kbar, bufs.scores, bufs.counts, bufs.cu, bufs.idx)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int32), bufs.scores.view(torch.int32))
    sc = before.cpu().numpy()
    banded = 0
    for (b, h, I, s, off) in segments(w.seqlens, w.hkv, w.block):
        row = sc[off:off + I + 1]
        th = np.float32(w.alpha) * row.max()
        J = np.arange(I + 1)
        free = (J >= w.sink) & (J < I - w.recent - w.window + 1)
        banded += int(((row >= th * np.float32(0.998)) & (row <= th * np.float32(1.002)) & free).any())
    log(f"[select] segments with a score in the uncertain band: {banded}")
    assert banded > 0


def test_deterministic_bitwise():
    w = GQA_BF16_16K.replace(seqlens=(4096,))
    inp = make_inputs(w, 0)
    dev = to_device(inp)
    a = run_gpu(w, inp, dev_tensors=dev)
    b = run_gpu(w, inp, dev_tensors=dev)
    for name in ("kbar", "scores", "idx", "out", "lse"):
        assert np.array_equal(getattr(a, name), getattr(b, name), equal_nan=True), name


# ----------------------------------------------------------------- full-size configs
#
# Every call passes the whole-array checks (run_gpu).  Every segment's
# scores and selection are compared with the oracle; attention outputs on
# every tile of one whole KV head plus sampled tiles of the others.

WORKERS = 16  # host threads for the oracle (the GPU machine's CPU share)


def _dense_error(w, inp, g, tiles):
    """Max-abs of the GPU's sparse output against exact dense causal attention
    (the oracle with every block selected), on the given tiles: the error the
    approximation itself makes, reported, not gated."""
    import oracle
    from harness import RequestView
    err = 0.0
    views = {}
    for (b, h, I) in sorted(tiles):
        if b not in views:
            views = {b: RequestView(w, inp, b)}
        rv = views[b]
        k_h, v_h, kbar_h, vbar_h = rv.head(h)
        pos, heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I, rv.q_off)
        O, _ = oracle.attend_rows(pos, rows, k_h, v_h, kbar_h, vbar_h, list(range(I + 1)), [],
                                  w.block, w.scale)
        go = g.out[rv.qstart + pos - rv.q_off, heads]
        err = max(err, float(np.abs(go - O).max()))
    return err


def _full_size(w, seed, rows=None, whole_head=None, per_head=3, dev=None, inp=None, **kw):
    from harness import compare_selection, oracle_score_rows
    inp = inp if inp is not None else make_inputs(w, seed)
    log(f"[parity] {w.name} seed={seed} {kw}: GPU run")
    g = run_gpu(w, inp, dev_tensors=dev, **kw)  # whole-array checks inside
    rows = rows if rows is not None else oracle_score_rows(w, inp, workers=WORKERS)
    sel = compare_selection(w, g, rows, alpha=kw.get("alpha"))
    log(f"[parity] {w.name} every segment: {sel}")
    assert sel.tiles == len(segments(w.seqlens, w.hkv, w.block, w.query_lens))
    assert sel.sel_mismatch == 0, str(sel)
    assert sel.score_rel < 5e-4, str(sel)
    tiles = sample_tiles(w, per_head=per_head, seed=seed)
    if whole_head is not None:
        for b, (L, Lq) in enumerate(zip(w.seqlens, w.query_lens)):
            N = -(-L // w.block)
            i0 = (L - Lq) // w.block if Lq else N
            tiles |= {(b, whole_head, I) for I in range(i0, N)}
    rep = compare(w, inp, g, tiles=tiles, workers=WORKERS, **kw)
    log(f"[parity] {w.name} attention tiles (KV head {whole_head} whole): {rep} gpu_ms={g.ms:.1f}")
    assert_parity(w, rep)
    return inp, g, rows, sel, rep


@pytest.mark.timeout(1200)
def test_sweep_64k_every_segment():
    # five alphas x correction on/off; scores do not depend on alpha, so the
    # oracle rows are computed once.  Per alpha: density, output error against
    # the oracle and against exact dense attention (correction on vs off).
    w = SWEEP_BF16_64K
    inp = make_inputs(w, 0)
    dev = to_device(inp)
    from harness import oracle_score_rows
    rows = oracle_score_rows(w, inp, workers=WORKERS)
    dense_tiles = sample_tiles(w, per_head=2, heads=[1])
    for a in SWEEP_ALPHAS:
        for corr in (True, False):
            whole = 3 if (a == 0.05 and corr) else None
            _, g, _, sel, rep = _full_size(w, 0, rows=rows, whole_head=whole, per_head=2, dev=dev,
                                           inp=inp, alpha=a, correction=corr)
            derr = _dense_error(w, inp, g, dense_tiles)
            log(f"[sweep] alpha={a} correction={corr} density={sel.selected / sel.blocks:.4f} "
                f"out_err_vs_oracle={rep.out_err:.3e} out_err_vs_dense={derr:.3e}")


@pytest.mark.timeout(1200)
def test_fp8_128k_every_segment():
    _full_size(FP8_128K, 0, whole_head=2)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("w", [SWEEP_BF16_64K, FP8_128K], ids=lambda w: w.name)
def test_full_size_second_seed(w):
    # the full-size workloads on fresh inputs (seed 1), as the bench runs them
    _full_size(w, 1, per_head=2)


def test_max_blocks_per_request_sampled():
    # the largest request the library takes: 16384 blocks of 64 tokens (1M
    # tokens, 1.3e8 score entries), which sizes the score kernel's per-block
    # maxima in LDS (64 KB), the attention's selection bitmap and the CSR at
    # their limits; g = 2 gives 128-row tiles
    w = Workload("max-blocks-1m-b64", (16384 * 64,), 2, 1, 64, 64, "bf16", attractors=4)
    inp = make_inputs(w, 0)
    g = run_gpu(w, inp)
    rep = compare(w, inp, g, tiles=sample_tiles(w, per_head=2))
    log(f"[parity] {w.name}: {rep} gpu_ms={g.ms:.1f}")
    assert_parity(w, rep)


@pytest.mark.timeout(1500)
def test_paged_varlen_6req_every_segment():
    _full_size(PAGED_VARLEN, 0, whole_head=5, per_head=2)


@pytest.mark.timeout(900)
def test_chunk_last_8k_of_64k_every_segment():
    # the chunked-prefill workload the bench times: 8K queries over 64K keys
    _full_size(CHUNK_BF16_64K, 0, whole_head=6, per_head=2)
