"""FP8 attention arithmetic of FlashPrefill V2, step by step, in float64.

Test infrastructure only (see the package docstring).

Source: "FlashPrefill V2" (paper text):
  * the FP8 paragraph: with per-tensor scales c_q, c_k, c_v the logits are
    S = c_q c_k (Q~ K~^T) * scale, the probabilities are rounded to e4m3 as
    P~ = e4m3(2^8 * exp(S - m)) with m the running row maximum, the output is
    O = c_v (P~ V~) / l, and the 2^8 offset is recovered in the log-sum-exp at
    finalize: LSE = m + ln l - 8 ln 2;
  * the CSR paragraph: the selected blocks are walked backwards, and under KV
    splitting split u of U takes a contiguous share of the CSR list balanced
    by count (Eq. 18);
  * the tile-configuration paragraph: key tiles of 64 columns, B/64 physical
    tiles per logical block;
  * Sec. 3.2 / Fig. 3 paragraph: pruned, fully visible blocks enter as extra
    iterations over pooled means with the score shifted by log|B_J|, grouped
    per chunk by a todo bitmask;
  * Tab. 8 paragraph: in FP8 the pooled statistics are quantised.
The partial results of the splits are merged with the online-softmax merge of
the PRR review page (Sec. 4.3, Eq. 6), `merge_partials`.

Readings taken where the pages leave a step open:
  * m is the exact running maximum: it is raised at every 64-key tile whose
    maximum exceeds it, and the accumulated numerator and l are rescaled;
  * a logical block's physical tiles are walked in descending order, as the
    blocks are (the dense schedule descends);
  * l sums the rounded probabilities P~ (numerator and denominator see the
    same values);
  * the correction terms come after the exact blocks, one step per chunk of
    64 pooled blocks that holds a todo block; the pooled means are quantised
    on the per-tensor scales of K and V: K-bar~ = e4m3(k-bar / c_k),
    V-bar~ = e4m3(v-bar / c_v), where k-bar / c_k is the exact mean of the
    block's codes (block means of codes often sit exactly on an e4m3
    midpoint; ties go to the even code);
  * with U splits, split u takes CSR positions [floor(u c / U),
    floor((u + 1) c / U)) of a list of c blocks and the correction chunks
    u, u + U, u + 2U, ...
"""
from __future__ import annotations

import math

import numpy as np

from .fp8 import decode_e4m3fn, encode_e4m3fn

TILE = 64   # keys per step (the pages' kBlockN)
CHUNK = 64  # pooled blocks per correction step
OFFSET = 2.0 ** 8


def e4m3_round(x):
    """Nearest e4m3 value (ties to even, saturating at 448), as float64."""
    return decode_e4m3fn(encode_e4m3fn(x))


def walk(sel, todo, B: int, L: int, u: int = 0, n_splits: int = 1):
    """Steps of split u: ("exact", key indices) for the physical tiles of its
    share of the ascending CSR list `sel`, walked backwards, then
    ("corr", blocks) for its correction chunks."""
    c = len(sel)
    beg, end = (u * c) // n_splits, ((u + 1) * c) // n_splits
    steps = []
    for t in range(end - 1, beg - 1, -1):
        J = sel[t]
        for h in range(B // TILE - 1, -1, -1):
            k0 = J * B + h * TILE
            if k0 < min((J + 1) * B, L):
                steps.append(("exact", np.arange(k0, min(k0 + TILE, (J + 1) * B, L))))
    todo = sorted(todo)
    n_chunks = max(todo) // CHUNK + 1 if todo else 0
    for ch in range(u, n_chunks, n_splits):
        blocks = [J for J in todo if ch * CHUNK <= J < (ch + 1) * CHUNK]
        if blocks:
            steps.append(("corr", blocks))
    return steps


def _rounding_neighbours(p):
    """The e4m3 values just below and just above each p (equal when p is on
    the grid)."""
    lo = e4m3_round(p)
    lo = np.where(lo > p, _step_down(lo), lo)
    hi = np.where(lo < p, _step_up(lo), lo)
    return lo, hi


def _step_down(x):
    codes = encode_e4m3fn(x).astype(np.int64)
    return decode_e4m3fn(np.maximum(codes - 1, 0).astype(np.uint8))


def _step_up(x):
    codes = encode_e4m3fn(x).astype(np.int64)
    return decode_e4m3fn(np.minimum(codes + 1, 0x7E).astype(np.uint8))


def pooled_code_means(x, scale: float, B: int):
    """Exact block means of the e4m3 codes of x = code * scale: the codes are
    recovered on their 2^-9 grid, and a mean of at most B such values is
    exact in float64."""
    codes = np.round(np.asarray(x, dtype=np.float64) / scale * 512.0) / 512.0
    L = codes.shape[0]
    return np.stack([codes[J * B:min((J + 1) * B, L)].mean(axis=0)
                     for J in range(-(-L // B))])


def attend_rows_fp8(pos, q_rows, k_h, v_h, sel, todo, B: int, scale: float, k_scale: float,
                    v_scale: float, n_splits: int = 1, quantize=e4m3_round, flips=(),
                    tie_band: float = 0.0):
    """Block-sparse causal attention with mean correction in the FP8
    arithmetic of the pages, for rows of one tile.

    q_rows, k_h, v_h are the dequantised inputs (code * scale); V~ = v_h /
    v_scale are the e4m3 codes.  The quantised pooled statistics are the e4m3
    rounding of the exact block means of the codes.  `quantize` rounds the
    probabilities and the pooled statistics; the identity gives exact
    arithmetic, which must equal `attend_rows`.

    Rounding near a tie.  A probability within `tie_band` (relative) of the
    midpoint between two e4m3 values may round either way in an
    implementation that computes its logits in lower precision; both results
    are correct roundings.  `flips` is a set of (row, key) whose probability
    is rounded to the other neighbour (key: token index, or ("pooled", J) for
    a corrected block).  With tie_band > 0 the near-tie keys are returned.

    Returns (O [rows, d], LSE [rows]) and, with tie_band > 0, a list per row
    of its near-tie keys.
    """
    L = k_h.shape[0]
    pos = np.asarray(pos)
    R, d = q_rows.shape
    kbar_q = quantize(pooled_code_means(k_h, k_scale, B)) * k_scale
    vbar_codes = quantize(pooled_code_means(v_h, v_scale, B))
    flips = set(flips)
    near = [[] for _ in range(R)]
    parts = []
    for u in range(n_splits):
        m = np.full(R, -np.inf)
        ell = np.zeros(R)
        acc = np.zeros((R, d))
        for kind, idx in walk(sel, todo, B, L, u, n_splits):
            if kind == "exact":
                x = scale * (q_rows @ k_h[idx].T)
                x = np.where(idx[None, :] <= pos[:, None], x, -np.inf)
                vals = v_h[idx] / v_scale
                keys = [int(j) for j in idx]
            else:
                size = np.array([min((J + 1) * B, L) - J * B for J in idx], dtype=np.float64)
                x = scale * (q_rows @ kbar_q[idx].T) + np.log(size)[None, :]
                vals = vbar_codes[idx]
                keys = [("pooled", int(J)) for J in idx]
            m_new = np.maximum(m, x.max(axis=1))
            grow = np.isfinite(m_new) & (m_new > m)
            keep = np.where(grow & np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) -
                                                          np.where(grow, m_new, 0.0)), 0.0)
            ell = np.where(grow, ell * keep, ell)
            acc = np.where(grow[:, None], acc * keep[:, None], acc)
            m = m_new
            ref = np.where(np.isfinite(m), m, 0.0)
            praw = OFFSET * np.exp(x - ref[:, None])
            p = quantize(praw)
            if flips or tie_band > 0:
                lo, hi = _rounding_neighbours(praw)
                mid = 0.5 * (lo + hi)
                col = {key: c for c, key in enumerate(keys)}
                for (r, key) in flips:
                    c = col.get(key)
                    if c is not None and lo[r, c] != hi[r, c]:
                        p[r, c] = lo[r, c] if p[r, c] == hi[r, c] else hi[r, c]
                if tie_band > 0:
                    close = (lo != hi) & (np.abs(praw - mid) <= tie_band * praw)
                    for r, c in zip(*np.nonzero(close)):
                        near[r].append(keys[c])
            ell = ell + p.sum(axis=1)
            acc = acc + p @ vals
        parts.append((acc, ell, m))
    # combine the splits (PRR review, Sec. 4.3, Eq. 6, over U partials): with
    # M = max_u m_u, each partial weighs l_u exp(m_u - M)
    ms = np.stack([np.where(e > 0, mu, -np.inf) for (_a, e, mu) in parts])
    M = ms.max(axis=0)
    seen = np.isfinite(M)
    Mr = np.where(seen, M, 0.0)
    num = np.zeros((R, d))
    ell = np.zeros(R)
    for (a_u, e_u, m_u) in parts:
        f = np.where(e_u > 0, np.exp(np.where(e_u > 0, m_u, 0.0) - Mr), 0.0)
        num += f[:, None] * a_u
        ell += f * e_u
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(seen[:, None], v_scale * num / np.where(seen, ell, 1.0)[:, None], 0.0)
        lse = np.where(seen, Mr + np.log(np.where(seen, ell, 1.0)) - math.log(OFFSET), -np.inf)
    if tie_band > 0:
        return O, lse, near
    return O, lse
