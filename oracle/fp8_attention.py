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
    V-bar~ = e4m3(v-bar / c_v);
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


def attend_rows_fp8(pos, q_rows, k_h, v_h, kbar_h, vbar_h, sel, todo, B: int, scale: float,
                    k_scale: float, v_scale: float, n_splits: int = 1, quantize=e4m3_round):
    """Block-sparse causal attention with mean correction in the FP8
    arithmetic of the pages, for rows of one tile.

    q_rows, k_h, v_h are the dequantised inputs (code * scale) and kbar_h,
    vbar_h the exact pooled means; V~ = v_h / v_scale are the e4m3 codes.
    `quantize` rounds the probabilities and the pooled statistics (e4m3);
    passing the identity gives exact arithmetic, which must equal
    `attend_rows`.  Returns (O [rows, d], LSE [rows]).
    """
    L = k_h.shape[0]
    pos = np.asarray(pos)
    R, d = q_rows.shape
    kbar_q = quantize(kbar_h / k_scale) * k_scale
    vbar_codes = quantize(vbar_h / v_scale)
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
            else:
                size = np.array([min((J + 1) * B, L) - J * B for J in idx], dtype=np.float64)
                x = scale * (q_rows @ kbar_q[idx].T) + np.log(size)[None, :]
                vals = vbar_codes[idx]
            m_new = np.maximum(m, x.max(axis=1))
            grow = np.isfinite(m_new) & (m_new > m)
            keep = np.where(grow & np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) -
                                                          np.where(grow, m_new, 0.0)), 0.0)
            ell = np.where(grow, ell * keep, ell)
            acc = np.where(grow[:, None], acc * keep[:, None], acc)
            m = m_new
            ref = np.where(np.isfinite(m), m, 0.0)
            p = quantize(OFFSET * np.exp(x - ref[:, None]))
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
    return O, lse
