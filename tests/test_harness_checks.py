"""CPU checks of the parity harness itself: the whole-array checks and the
every-segment selection comparison accept a result built from the oracle and
reject results with a planted defect (a missed write, an unsorted or
out-of-range index list, a count that disagrees with cu, a flipped block).
No GPU: the "device" result here is assembled from oracle outputs."""
import numpy as np
import pytest

import oracle
from harness import (GpuResult, Report, check_arrays, compare_selection, oracle_score_rows,
                     segment_arrays, segments)
from workloads import Workload, make_inputs


def _oracle_result(w, inp) -> GpuResult:
    """A result in the C-ABI layout filled from the oracle, request by request."""
    from harness import RequestView
    segs = segments(w.seqlens, w.hkv, w.block, w.query_lens)
    n_sc = sum(I + 1 for (_b, _h, I, _s, _o) in segs)
    pooled = sum(-(-L // w.block) for L in w.seqlens)
    T = sum(w.query_lens)
    kbar = np.zeros((pooled, w.hkv, w.d), np.float32)
    vbar = np.zeros_like(kbar)
    scores = np.zeros(max(1, n_sc), np.float32)
    counts = np.zeros(max(1, len(segs)), np.int32)
    out = np.zeros((T, w.hq, w.d), np.float32)
    lse = np.zeros((w.hq, T), np.float32)
    sels = []
    pb = 0
    for b, L in enumerate(w.seqlens):
        rv = RequestView(w, inp, b)
        N = -(-L // w.block)
        for h in range(w.hkv):
            k_h, v_h, kb, vb = rv.head(h)
            kbar[pb:pb + N, h] = kb
            vbar[pb:pb + N, h] = vb
        for (bb, h, I, s, off) in segs:
            if bb != b:
                continue
            k_h, v_h, kb, vb = rv.head(h)
            pos, heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I, rv.q_off)
            sc = oracle.block_scores_row(rows, kb, I, w.scale)
            sel, _ = oracle.select_row(sc, I, w.alpha, w.sink, w.window, w.recent)
            scores[off:off + I + 1] = sc
            counts[s] = len(sel)
            sels.append((s, sel))
            O, l = oracle.attend_rows(pos, rows, k_h, v_h, kb, vb, sel,
                                      oracle.todo_row(sel, I, w.correction), w.block, w.scale)
            out[rv.qstart + pos - rv.q_off, heads] = O
            lse[heads, rv.qstart + pos - rv.q_off] = l
        pb += N
    cu = np.concatenate([[0], np.cumsum(counts[:len(segs)])]).astype(np.int32)
    idx = np.full(max(1, n_sc), -7, np.int32)
    for s, sel in sels:
        idx[cu[s]:cu[s] + len(sel)] = sel
    return GpuResult(kbar, vbar, scores, counts, cu, idx, out, lse)


W = Workload("harness-self-check", (700, 300), 8, 2, 64, 64, "bf16", attractors=3)


@pytest.fixture(scope="module")
def fixture():
    inp = make_inputs(W, 4)
    return inp, _oracle_result(W, inp)


def _copy(g):
    return GpuResult(*(np.array(getattr(g, f), copy=True) for f in
                       ("kbar", "vbar", "scores", "counts", "cu", "idx", "out", "lse")))


def test_oracle_result_passes(fixture):
    inp, g = fixture
    check_arrays(W, g)
    rows = oracle_score_rows(W, inp, workers=2)
    rep = compare_selection(W, g, rows)
    assert rep.tiles == len(segment_arrays(W)[0])
    assert rep.sel_mismatch == 0 and rep.score_rel < 1e-6


@pytest.mark.parametrize("defect", ["nan_out", "nan_score", "nan_lse", "unsorted", "range",
                                    "counts", "not_diagonal"])
def test_defects_are_caught(fixture, defect):
    _inp, g0 = fixture
    g = _copy(g0)
    if defect == "nan_out":
        g.out[g.out.shape[0] - 1, 3, 5] = np.nan
    elif defect == "nan_score":
        g.scores[len(g.scores) // 2] = np.nan
    elif defect == "nan_lse":
        g.lse[1, 7] = np.nan
    elif defect == "unsorted":
        s = int(np.argmax(g.counts >= 3))
        a = int(g.cu[s])
        g.idx[a], g.idx[a + 1] = g.idx[a + 1], g.idx[a]
    elif defect == "range":
        s = int(np.argmax(g.counts >= 2))
        g.idx[int(g.cu[s])] = -7
    elif defect == "counts":
        g.counts[3] += 1
    elif defect == "not_diagonal":
        s = len(segment_arrays(W)[0]) - 1
        g.idx[int(g.cu[s + 1]) - 1] -= 1
    with pytest.raises(AssertionError):
        check_arrays(W, g)


def test_flipped_block_is_counted(fixture):
    inp, g0 = fixture
    g = _copy(g0)
    rows = oracle_score_rows(W, inp, workers=2)
    # drop a non-forced selected block of some segment (its count and cu move with it)
    _b, _h, I, _off = segment_arrays(W)
    for s in range(len(I)):
        sel = list(g.idx[g.cu[s]:g.cu[s + 1]])
        forced = oracle.forced_blocks(int(I[s]), W.sink, W.window, W.recent)
        extra = [J for J in sel if J not in forced]
        if extra:
            break
    else:
        pytest.skip("no thresholded block in this workload")
    keep = [J for J in sel if J != extra[0]]
    tail = list(g.idx[g.cu[s + 1]:g.cu[-1]])
    g.idx[g.cu[s]:g.cu[s] + len(keep)] = keep
    g.idx[g.cu[s] + len(keep):g.cu[s] + len(keep) + len(tail)] = tail
    g.counts[s] -= 1
    g.cu[s + 1:] -= 1
    check_arrays(W, g)  # still a valid CSR
    rep = compare_selection(W, g, rows)
    assert rep.sel_mismatch == 1
