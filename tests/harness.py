"""Test infrastructure: run the HIP pipeline on seeded inputs and compare it
with the fp64 oracle tile by tile.  Imports the product binding and the
oracle side by side; neither imports the other."""
from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass

import numpy as np

import oracle
from workloads import Workload, make_inputs

SEL_BAND = 1e-5  # blocks with |Score - thresh| <= SEL_BAND * thresh may go either way


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def segments(seqlens, hkv, B, q_lens=None):
    """(b, h, I, segment index, score offset) in the C-ABI layout of bslp.h:
    per request the tiles I >= i0 that hold a query, I + 1 scores each."""
    q_lens = seqlens if q_lens is None else q_lens
    out = []
    seg = 0
    sc = 0
    for b, (L, Lq) in enumerate(zip(seqlens, q_lens)):
        N = -(-L // B)
        i0 = (L - Lq) // B if Lq else N
        first = i0 * (i0 + 1) // 2
        tri = N * (N + 1) // 2 - first
        for h in range(hkv):
            for I in range(i0, N):
                out.append((b, h, I, seg + h * (N - i0) + I - i0, sc + h * tri + I * (I + 1) // 2 - first))
        seg += hkv * (N - i0)
        sc += hkv * tri
    return out


@dataclass
class GpuResult:
    kbar: np.ndarray
    vbar: np.ndarray
    scores: np.ndarray
    counts: np.ndarray
    cu: np.ndarray
    idx: np.ndarray
    out: np.ndarray
    lse: np.ndarray
    ms: float = 0.0


def to_device(inp):
    import torch
    dev = torch.device("cuda")
    table = None
    if inp.table is not None:
        table = torch.from_numpy(inp.table).to(dev)
    return inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), table


def run_gpu(w: Workload, inp, alpha=None, correction=None, dev_tensors=None,
            kv_splits: int = 0) -> GpuResult:
    import torch

    import block_sparse_long_pooled_amd as bslp
    q, k, v, table = dev_tensors or to_device(inp)
    prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.query_lens,
                             softmax_scale=w.scale, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             v_scale=inp.v_scale, page_table=table, page_size=w.page_size,
                             kv_splits=kv_splits,
                             kv_seqlens=w.seqlens if w.q_lens is not None else None)
    params = bslp.make_params(w.alpha if alpha is None else alpha, w.sink, w.window, w.recent,
                              w.correction if correction is None else correction)
    bufs = bslp.Buffers(prob)
    # poison every output so a missed write shows up
    for t in (bufs.kbar, bufs.vbar, bufs.scores, bufs.lse):
        t.fill_(float("nan"))
    for t in (bufs.counts, bufs.cu, bufs.idx):
        t.fill_(-7)
    bufs.out.fill_(float("nan"))
    torch.cuda.synchronize()
    t0 = time.time()
    bslp.prefill(prob, params, q, k, v, bufs)
    torch.cuda.synchronize()
    ms = (time.time() - t0) * 1e3
    c = lambda t: t.cpu().numpy()
    return GpuResult(c(bufs.kbar), c(bufs.vbar), c(bufs.scores), c(bufs.counts), c(bufs.cu),
                     c(bufs.idx), c(bufs.out.float()), c(bufs.lse), ms)


def dequant(t, scale: float, dtype: str) -> np.ndarray:
    """Exactly the values the GPU reads, as float32 (bf16 and e4m3 widen exactly)."""
    import torch
    if dtype == "fp8":
        return (oracle.decode_e4m3fn(t.numpy()) * scale).astype(np.float64)
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


class RequestView:
    """Oracle-side arrays of one request, built lazily (float64 per KV head)."""

    def __init__(self, w: Workload, inp, b: int):
        self.w = w
        start = sum(w.seqlens[:b])
        L = w.seqlens[b]
        self.L = L
        qstart, Lq = sum(w.query_lens[:b]), w.query_lens[b]
        self.q_off = L - Lq
        self.qstart = qstart
        kk = inp.k_logical if inp.k_logical is not None else inp.k
        vv = inp.v_logical if inp.v_logical is not None else inp.v
        self.q = dequant(inp.q[qstart:qstart + Lq], inp.q_scale, w.dtype)
        self._k = kk[start:start + L]
        self._v = vv[start:start + L]
        self.ks, self.vs = inp.k_scale, inp.v_scale
        self._heads = {}

    def head(self, h):
        if h not in self._heads:
            k = dequant(self._k[:, h:h + 1].contiguous(), self.ks, self.w.dtype).astype(np.float64)
            v = dequant(self._v[:, h:h + 1].contiguous(), self.vs, self.w.dtype).astype(np.float64)
            kbar = oracle.pool_means(k, self.w.block)[:, 0]
            vbar = oracle.pool_means(v, self.w.block)[:, 0]
            self._heads[h] = (k[:, 0], v[:, 0], kbar, vbar)
        return self._heads[h]


def out_tol(dtype: str) -> float:
    return 2e-3 if dtype == "f32" else 2e-2


class Report:
    def __init__(self):
        self.tiles = 0
        self.sel_mismatch = 0
        self.band = 0
        self.score_rel = 0.0
        self.kbar_err = 0.0
        self.out_err = 0.0
        self.lse_err = 0.0
        self.blocks = 0
        self.selected = 0

    def __str__(self):
        return (f"tiles={self.tiles} sel_mismatch={self.sel_mismatch} band={self.band} "
                f"score_rel={self.score_rel:.2e} pooled_err={self.kbar_err:.2e} "
                f"out_maxabs={self.out_err:.3e} lse_maxabs={self.lse_err:.3e} "
                f"density={self.selected / max(1, self.blocks):.4f}")


def compare(w: Workload, inp, g: GpuResult, tiles=None, alpha=None, correction=None,
            rep: Report | None = None) -> Report:
    """Compare GPU results with the oracle on every (or the chosen) tiles.

    tiles: None for all, or a set of (b, h, I)."""
    rep = rep or Report()
    alpha = w.alpha if alpha is None else alpha
    corr = w.correction if correction is None else correction
    segs = segments(w.seqlens, w.hkv, w.block, w.query_lens)
    views = {}
    pool_bases = np.concatenate([[0], np.cumsum([-(-L // w.block) for L in w.seqlens])])
    for (b, h, I, s, off) in segs:
        if tiles is not None and (b, h, I) not in tiles:
            continue
        if b not in views:
            views = {b: RequestView(w, inp, b)}
        rv = views[b]
        k_h, v_h, kbar_h, vbar_h = rv.head(h)
        N = kbar_h.shape[0]
        pb = pool_bases[b]
        # pooled means
        rep.kbar_err = max(rep.kbar_err, float(np.abs(g.kbar[pb:pb + N, h] - kbar_h).max()),
                           float(np.abs(g.vbar[pb:pb + N, h] - vbar_h).max()))
        # scores
        pos, heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I, rv.q_off)
        score = oracle.block_scores_row(rows, kbar_h, I, w.scale)
        sel_o, thresh = oracle.select_row(score, I, alpha, w.sink, w.window, w.recent)
        gs = g.scores[off:off + I + 1].astype(np.float64)
        big = score > 1e-30
        if big.any():
            rep.score_rel = max(rep.score_rel, float((np.abs(gs[big] - score[big]) / score[big]).max()))
        assert np.all(np.isfinite(gs)), f"non-finite score in segment {(b, h, I)}"
        # selection: bit-exact outside the band, valid inside it
        beg, end = int(g.cu[s]), int(g.cu[s + 1])
        assert end - beg == int(g.counts[s]), f"count/cu mismatch at {(b, h, I)}"
        sel_g = [int(x) for x in g.idx[beg:end]]
        assert sel_g == sorted(set(sel_g)), f"unsorted/duplicate selection at {(b, h, I)}"
        assert all(0 <= J <= I for J in sel_g)
        forced = oracle.forced_blocks(I, w.sink, w.window, w.recent)
        assert forced <= set(sel_g), f"forced block missing at {(b, h, I)}"
        so, sg = set(sel_o), set(sel_g)
        for J in range(I + 1):
            in_band = J not in forced and abs(score[J] - thresh) <= SEL_BAND * thresh
            if in_band:
                rep.band += 1
            elif (J in so) != (J in sg):
                rep.sel_mismatch += 1
        rep.blocks += I + 1
        rep.selected += len(sel_g)
        # attention on the (validated) GPU selection
        todo = oracle.todo_row(sel_g, I, corr)
        O, lse = oracle.attend_rows(pos, rows, k_h, v_h, kbar_h, vbar_h, sel_g, todo, w.block,
                                    w.scale)
        go = g.out[rv.qstart + pos - rv.q_off, heads]
        gl = g.lse[heads, rv.qstart + pos - rv.q_off]
        rep.out_err = max(rep.out_err, float(np.abs(go - O).max()))
        fin = np.isfinite(lse)
        assert np.array_equal(fin, np.isfinite(gl)), f"LSE finiteness differs at {(b, h, I)}"
        if fin.any():
            rep.lse_err = max(rep.lse_err, float(np.abs(gl[fin] - lse[fin]).max()))
        rep.tiles += 1
    return rep


def assert_parity(w: Workload, rep: Report):
    assert rep.tiles > 0
    assert rep.sel_mismatch == 0, str(rep)
    assert rep.score_rel < 1e-4, str(rep)
    assert rep.kbar_err < 1e-4, str(rep)
    assert rep.out_err <= out_tol(w.dtype), str(rep)
    assert rep.lse_err <= (1e-3 if w.dtype == "f32" else 2e-2), str(rep)


def sample_tiles(w: Workload, per_head: int = 4, heads=None, seed: int = 0):
    """The first, second, middle, last tiles plus a few random ones per
    sampled head, for every request."""
    rng = np.random.default_rng(seed)
    heads = heads if heads is not None else sorted({0, w.hkv - 1})
    out = set()
    for b, (L, Lq) in enumerate(zip(w.seqlens, w.query_lens)):
        N = -(-L // w.block)
        if Lq == 0:
            continue
        i0 = (L - Lq) // w.block  # tiles that hold a query
        span = N - i0
        for h in heads:
            for I in {0, 1 % span, span // 2, span - 1, *rng.integers(0, span, per_head).tolist()}:
                out.add((b, h, i0 + int(I)))
    return out


def dense_flops(w: Workload) -> float:
    return 4.0 * w.d * w.hq * sum(L * (L + 1) / 2 for L in w.seqlens)


__all__ = ["GpuResult", "Report", "assert_parity", "compare", "dense_flops", "log",
           "make_inputs", "run_gpu", "sample_tiles", "segments", "to_device", "math"]
