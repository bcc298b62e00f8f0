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
    kv_splits: int = 0  # the launch's kv_splits request (0: automatic)


def to_device(inp):
    import torch
    dev = torch.device("cuda")
    table = None
    if inp.table is not None:
        table = torch.from_numpy(inp.table).to(dev)
    return inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), table


def v_dmajor(w: Workload, v):
    """V in the d-major layout of the C ABI: [Hkv, d, kv tokens] from [tokens,
    Hkv, d], or [pages, Hkv, d, page] from the paged [pages * page, Hkv, d]."""
    if w.page_size:
        p = w.page_size
        return v.reshape(-1, p, w.hkv, w.d).permute(0, 2, 3, 1).contiguous()
    return v.permute(1, 2, 0).contiguous()


def run_gpu(w: Workload, inp, alpha=None, correction=None, dev_tensors=None,
            kv_splits: int = 0, check: bool = True, v_dmajor: bool = False) -> GpuResult:
    """One prefill through the C ABI on poisoned output buffers; with `check`
    the whole-array checks (check_arrays) run on the result."""
    import torch

    import block_sparse_long_pooled_amd as bslp
    q, k, v, table = dev_tensors or to_device(inp)
    prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.query_lens,
                             softmax_scale=w.scale, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             v_scale=inp.v_scale, page_table=table, page_size=w.page_size,
                             kv_splits=kv_splits,
                             kv_seqlens=w.seqlens if w.q_lens is not None else None,
                             v_dmajor=v_dmajor)
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
    res = GpuResult(c(bufs.kbar), c(bufs.vbar), c(bufs.scores), c(bufs.counts), c(bufs.cu),
                    c(bufs.idx), c(bufs.out.float()), c(bufs.lse), ms, kv_splits)
    if check:
        check_arrays(w, res)
    return res


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

    def drop_head(self, h):
        """Frees the token-level K/V of head h, keeping its pooled means."""
        if h in self._heads:
            _k, _v, kbar, vbar = self._heads[h]
            self._heads[h] = (None, None, kbar, vbar)


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
        self.exact_err = 0.0  # fp8: output against exact (unrounded) arithmetic, not gated
        self.tie_rows = 0     # fp8: rows matched with another rounding of a near tie
        self.blocks = 0
        self.selected = 0

    def merge(self, o: "Report"):
        self.tiles += o.tiles
        self.sel_mismatch += o.sel_mismatch
        self.band += o.band
        self.blocks += o.blocks
        self.selected += o.selected
        self.tie_rows += o.tie_rows
        for f in ("score_rel", "kbar_err", "out_err", "lse_err", "exact_err"):
            setattr(self, f, max(getattr(self, f), getattr(o, f)))

    def __str__(self):
        return (f"tiles={self.tiles} sel_mismatch={self.sel_mismatch} band={self.band} "
                f"score_rel={self.score_rel:.2e} pooled_err={self.kbar_err:.2e} "
                f"out_maxabs={self.out_err:.3e} lse_maxabs={self.lse_err:.3e} "
                f"density={self.selected / max(1, self.blocks):.4f}" +
                (f" out_vs_exact={self.exact_err:.3e} tie_rows={self.tie_rows}"
                 if self.exact_err else ""))


def launch_split_allowance(w: Workload, kv_splits: int) -> int:
    """KV splits a launch allows, by the rule bslp.h documents for
    bslp_problem.kv_splits: 1 for float32 or kv_splits = 1; kv_splits when
    2..16; automatic (0): when the launch has fewer than 512 work units (of
    256, 128 or 64 packed rows) and some request has at least 16 blocks,
    ceil(512 / units) capped at 4, else 1."""
    if w.dtype == "f32" or kv_splits == 1:
        return 1
    if kv_splits >= 2:
        return kv_splits
    rows = w.g * w.block
    per_unit = 256 if rows >= 256 else 128 if rows >= 128 else 64
    ups = -(-rows // per_unit)
    tiles = 0
    max_n = 0
    for L, Lq in zip(w.seqlens, w.query_lens):
        N = -(-L // w.block)
        i0 = (L - Lq) // w.block if Lq else N
        tiles += N - i0
        max_n = max(max_n, N)
    units = tiles * w.hkv * ups
    if units == 0 or units >= 512 or max_n < 16:
        return 1
    return min(4, -(-512 // units))


def segment_splits(n_sel: int, I: int, B: int, correction: bool, allowance: int) -> int:
    """Splits of one segment (bslp.h): one per 24 steps of work, its selected
    blocks in 64-key tiles plus its correction chunks, at most `allowance`."""
    steps = n_sel * (B // 64) + ((I + 63) // 64 if correction and I > 0 else 0)
    return max(1, min(allowance, steps // 24))


# A probability within this relative distance of an e4m3 rounding midpoint may
# round either way on the GPU: its logits carry float32 rounding (values up
# to about 2^7 in log2 units, an ulp of 7.6e-6, so P moves by about 5e-6),
# the matrix cores' float32 accumulation and v_exp_f32's last-bit error.
# 1e-4 is twenty times that.  Both roundings are correct results.
FP8_TIE_BAND = 1e-4


def _resolve_ties(w, rv, pos, rows, k_h, v_h, sel, todo, ns, go, gl, O, lse, near, rep):
    """Rows whose GPU output misses the oracle's and that hold near-tie
    probabilities are compared with the oracle's other roundings of those
    (at most the 3 heaviest, every subset); the closest is kept."""
    import itertools
    tol = out_tol(w.dtype)
    err = np.abs(go - O).max(axis=1)
    fin = np.isfinite(lse)
    lerr = np.where(fin, np.abs(np.where(fin, gl - lse, 0.0)), 0.0)
    O, lse = O.copy(), lse.copy()
    for r in np.nonzero((err > tol) | (lerr > 2e-2))[0]:
        if not near[r]:
            continue
        keys = near[r][-3:]
        best = (err[r], O[r], lse[r])
        for n in range(1, len(keys) + 1):
            for sub in itertools.combinations(keys, n):
                Or, lr = oracle.attend_rows_fp8([pos[r]], rows[r:r + 1], k_h, v_h, sel, todo,
                                                w.block, w.scale, rv.ks, rv.vs, n_splits=ns,
                                                flips={(0, key) for key in sub})
                e = float(np.abs(go[r] - Or[0]).max())
                if e < best[0]:
                    best = (e, Or[0], lr[0])
        if best[0] < err[r]:
            O[r], lse[r] = best[1], best[2]
            rep.tie_rows += 1
    return O, lse


def _tile_check(w, rv, b, h, I, s, off, g: GpuResult, alpha, corr, pb, rep: Report):
    """Oracle vs GPU on one tile: pooled means of the head, score row,
    selection (bit-exact outside the band), attention rows on the GPU's
    validated selection."""
    k_h, v_h, kbar_h, vbar_h = rv.head(h)
    N = kbar_h.shape[0]
    rep.kbar_err = max(rep.kbar_err, float(np.abs(g.kbar[pb:pb + N, h] - kbar_h).max()),
                       float(np.abs(g.vbar[pb:pb + N, h] - vbar_h).max()))
    pos, heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I, rv.q_off)
    score = oracle.block_scores_row(rows, kbar_h, I, w.scale)
    sel_o, thresh = oracle.select_row(score, I, alpha, w.sink, w.window, w.recent)
    gs = g.scores[off:off + I + 1].astype(np.float64)
    assert np.all(np.isfinite(gs)), f"non-finite score in segment {(b, h, I)}"
    big = score > 1e-30
    if big.any():
        rep.score_rel = max(rep.score_rel, float((np.abs(gs[big] - score[big]) / score[big]).max()))
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
    todo = oracle.todo_row(sel_g, I, corr)
    if w.dtype == "fp8":
        # the FP8 arithmetic of the pages (e4m3 probabilities against the
        # running maximum of the walk, quantised pooled statistics), over the
        # splits the launch gave this segment
        ns = segment_splits(len(sel_g), I, w.block, corr,
                            launch_split_allowance(w, g.kv_splits))
        O, lse, near = oracle.attend_rows_fp8(pos, rows, k_h, v_h, sel_g, todo, w.block, w.scale,
                                              rv.ks, rv.vs, n_splits=ns, tie_band=FP8_TIE_BAND)
        go = g.out[rv.qstart + pos - rv.q_off, heads]
        gl = g.lse[heads, rv.qstart + pos - rv.q_off]
        O, lse = _resolve_ties(w, rv, pos, rows, k_h, v_h, sel_g, todo, ns, go, gl, O, lse, near,
                               rep)
        Ox, _ = oracle.attend_rows(pos, rows, k_h, v_h, kbar_h, vbar_h, sel_g, todo, w.block,
                                   w.scale)
        rep.exact_err = max(rep.exact_err, float(np.abs(go - Ox).max()))
    else:
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


def _blas_single_thread():
    """Context that pins BLAS to one thread while worker threads run oracle
    tiles side by side (numpy releases the GIL inside its kernels)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1, user_api="blas")
    except Exception:  # noqa: BLE001
        import contextlib
        return contextlib.nullcontext()


def compare(w: Workload, inp, g: GpuResult, tiles=None, alpha=None, correction=None,
            rep: Report | None = None, workers: int = 1) -> Report:
    """Compare GPU results with the oracle on every (or the chosen) tiles.

    tiles: None for all, or a set of (b, h, I).  workers > 1 runs the
    (request, KV head) groups in parallel threads."""
    rep = rep or Report()
    alpha = w.alpha if alpha is None else alpha
    corr = w.correction if correction is None else correction
    segs = segments(w.seqlens, w.hkv, w.block, w.query_lens)
    pool_bases = np.concatenate([[0], np.cumsum([-(-L // w.block) for L in w.seqlens])])
    groups: dict = {}
    for (b, h, I, s, off) in segs:
        if tiles is None or (b, h, I) in tiles:
            groups.setdefault((b, h), []).append((I, s, off))
    if workers <= 1:
        views = {}
        for (b, h), items in groups.items():
            if b not in views:
                views = {b: RequestView(w, inp, b)}  # one request's arrays at a time
            for (I, s, off) in items:
                _tile_check(w, views[b], b, h, I, s, off, g, alpha, corr, pool_bases[b], rep)
        return rep
    views = {b: RequestView(w, inp, b) for b in sorted({b for b, _ in groups})}
    from concurrent.futures import ThreadPoolExecutor
    # jobs: slices of a group's tiles, about 4 per worker, heaviest tiles
    # spread over the slices; each head's arrays are built once beforehand
    jobs = []
    n_items = sum(len(v) for v in groups.values())
    per_job = max(1, n_items // (4 * workers))
    for key, items in groups.items():
        for j0 in range(0, len(items), per_job):
            jobs.append((key, items[j0:j0 + per_job]))

    def run(job):
        (b, h), items = job
        r = Report()
        for (I, s, off) in items:
            _tile_check(w, views[b], b, h, I, s, off, g, alpha, corr, pool_bases[b], r)
        return r

    with _blas_single_thread(), ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda key: views[key[0]].head(key[1]), list(groups)))
        for r in ex.map(run, jobs):
            rep.merge(r)
    return rep


def segment_arrays(w: Workload):
    """Per segment, in C-ABI order: request, KV head, tile I and score offset
    (numpy arrays)."""
    segs = segments(w.seqlens, w.hkv, w.block, w.query_lens)
    a = np.array([(b, h, I, off) for (b, h, I, _s, off) in segs], dtype=np.int64).reshape(-1, 4)
    return a[:, 0], a[:, 1], a[:, 2], a[:, 3]


def check_arrays(w: Workload, g: GpuResult):
    """Whole-array checks of one call, cheap at any size: no poison (NaN or
    -7) left in any output, counts == diff(cu), every CSR list strictly
    ascending inside [0, I] and ending at the diagonal block when recent
    blocks are forced, every LSE finite when every row sees a key."""
    _b, _h, I, _off = segment_arrays(w)
    nseg = I.shape[0]
    n_sc = int((I + 1).sum())  # one score (and idx slot) per block J <= I of a segment
    assert np.isfinite(g.kbar).all() and np.isfinite(g.vbar).all(), "pooled means not finite"
    assert np.isfinite(g.scores[:n_sc]).all(), "a score is not finite (missed write?)"
    cu = g.cu.astype(np.int64)
    counts = g.counts[:nseg].astype(np.int64)
    assert cu[0] == 0 and np.array_equal(np.diff(cu[:nseg + 1]), counts), "counts != diff(cu)"
    if nseg:
        assert (counts >= (1 if w.recent >= 1 else 0)).all(), "a segment lost its diagonal block"
    total = int(cu[nseg])
    assert total <= n_sc, "CSR longer than its capacity"
    idx = g.idx[:total].astype(np.int64)
    seg_of = np.repeat(np.arange(nseg), counts)
    assert (idx >= 0).all() and (idx <= I[seg_of]).all(), "CSR index outside [0, I]"
    same = seg_of[1:] == seg_of[:-1]
    assert (idx[1:][same] > idx[:-1][same]).all(), "CSR list not strictly ascending"
    if w.recent >= 1 and nseg:
        assert np.array_equal(idx[cu[1:nseg + 1] - 1], I), "a CSR list does not end at I"
    rows = g.out.shape[0]
    for r0 in range(0, rows, 1 << 14):  # chunked: the output can be GBs
        assert np.isfinite(g.out[r0:r0 + (1 << 14)]).all(), f"non-finite output in rows {r0}.."
    assert not np.isnan(g.lse).any(), "NaN left in the LSE"
    if w.recent >= 1:
        assert np.isfinite(g.lse).all(), "an LSE is not finite though every row sees a key"


def oracle_score_rows(w: Workload, inp, workers: int = 8, heads=None) -> dict:
    """Oracle score rows of every segment (optionally of some KV heads only):
    {(b, h): [row of tile I for I = i0 .. N-1]}."""
    from concurrent.futures import ThreadPoolExecutor
    heads = range(w.hkv) if heads is None else heads
    views = {b: RequestView(w, inp, b) for b, Lq in enumerate(w.query_lens) if Lq}
    keys = [(b, h) for b in views for h in heads]

    def pooled(key):
        b, h = key
        kbar_h = views[b].head(h)[2]
        views[b].drop_head(h)  # keep only the pooled means of this head
        return key, kbar_h

    def run(job):
        (b, h), kbar_h, I_lo, I_hi = job
        rv = views[b]
        out = []
        for I in range(I_lo, I_hi):
            _pos, _heads, rows = oracle.tile_query_rows(rv.q, h, w.g, w.block, I, rv.q_off)
            out.append(oracle.block_scores_row(rows, kbar_h, I, w.scale))
        return (b, h), I_lo, out

    with _blas_single_thread(), ThreadPoolExecutor(max_workers=workers) as ex:
        kbars = dict(ex.map(pooled, keys))
        # tile ranges of about equal work (a tile's cost grows with I + 1),
        # about 4 per worker over all heads
        work = {key: np.cumsum(np.arange(views[key[0]].q_off // w.block, kb.shape[0]) + 1.0)
                for key, kb in kbars.items()}
        total = sum(float(c[-1]) for c in work.values() if c.size)
        jobs = []
        for key, c in work.items():
            if not c.size:
                continue
            i0 = views[key[0]].q_off // w.block
            parts = max(1, min(c.size, int(np.ceil(4 * workers * c[-1] / total))))
            cuts = np.searchsorted(c, c[-1] * np.arange(1, parts) / parts)
            bounds = [i0] + [i0 + int(x) for x in cuts] + [i0 + c.size]
            jobs += [(key, kbars[key], lo, hi) for lo, hi in zip(bounds[:-1], bounds[1:]) if hi > lo]
        rows_by = {}
        for key, lo, out in ex.map(run, jobs):
            rows_by.setdefault(key, []).append((lo, out))
    return {key: [r for _lo, part in sorted(parts) for r in part] for key, parts in rows_by.items()}


def compare_selection(w: Workload, g: GpuResult, rows: dict, alpha=None) -> Report:
    """Scores and selection of every segment whose oracle row is in `rows`
    (from oracle_score_rows) against the GPU's: the selection bit-exact
    outside the 1e-5 band of thresh_I, the forced blocks present."""
    alpha = w.alpha if alpha is None else alpha
    rep = Report()
    b_a, h_a, I_a, off_a = segment_arrays(w)
    i0 = {b: ((L - Lq) // w.block if Lq else 0) for b, (L, Lq) in
          enumerate(zip(w.seqlens, w.query_lens))}
    cu = g.cu.astype(np.int64)
    for s in range(I_a.shape[0]):
        b, h, I, off = int(b_a[s]), int(h_a[s]), int(I_a[s]), int(off_a[s])
        if (b, h) not in rows:
            continue
        score = rows[(b, h)][I - i0[b]]
        gs = g.scores[off:off + I + 1].astype(np.float64)
        big = score > 1e-30
        if big.any():
            rep.score_rel = max(rep.score_rel,
                                float((np.abs(gs[big] - score[big]) / score[big]).max()))
        thresh = alpha * score.max()
        keep_o = score >= thresh
        forced = np.zeros(I + 1, dtype=bool)
        forced[sorted(oracle.forced_blocks(I, w.sink, w.window, w.recent))] = True
        keep_o |= forced
        keep_g = np.zeros(I + 1, dtype=bool)
        keep_g[g.idx[cu[s]:cu[s + 1]]] = True
        assert keep_g[forced].all(), f"forced block missing at {(b, h, I)}"
        band = ~forced & (np.abs(score - thresh) <= SEL_BAND * thresh)
        rep.band += int(band.sum())
        rep.sel_mismatch += int(((keep_o != keep_g) & ~band).sum())
        rep.blocks += I + 1
        rep.selected += int(keep_g.sum())
        rep.tiles += 1
    return rep


def assert_parity(w: Workload, rep: Report):
    assert rep.tiles > 0
    assert rep.sel_mismatch == 0, str(rep)
    # the selection re-decides blocks within 2 x 1e-3 of the threshold exactly,
    # which assumes score errors below 1e-3; half of it leaves a margin
    assert rep.score_rel < 5e-4, str(rep)
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


__all__ = ["GpuResult", "Report", "assert_parity", "check_arrays", "compare",
           "launch_split_allowance", "segment_splits",
           "compare_selection", "dense_flops", "log", "make_inputs", "oracle_score_rows",
           "run_gpu", "sample_tiles", "segment_arrays", "segments", "to_device", "math"]
