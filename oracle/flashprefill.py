"""Float64 oracle of the FlashPrefill / FlashPrefill V2 prefill hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, cited by page title and section:
  [V2]  "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
        Serving" (paper text): Sec. 3.1 (mean-pooled keys, fused block scores,
        max-based threshold, sink/window/recent blocks), Sec. 3.2 (mean
        correction, Eq. 6 / Eq. 8 / Eq. 9 and the Fig. 3 correction path),
        the PackGQA paragraph, the FP8 paragraph and the CSR paragraph.
  [V1]  "FlashPrefill: Instantaneous Pattern Discovery and Thresholding for
        Ultra-Fast Long-Context Prefilling" (summary page), method-steps
        section, where the block-score and threshold formulas are printed.
  [PRR] the PRR (Predict, Reuse, Repair) review page, Sec. 4.3, Eq. 6: the
        online-softmax merge recurrence.

Readings taken where the pages are silent:
  * logits carry the softmax scale in scoring and in attention;
  * scoring is block-causal (J <= I) with no token mask inside the diagonal
    block;
  * under GQA one selection is made per (request, KV head, tile I); the tile's
    rows are its B positions times the g query heads of that KV head;
  * sink / window / recent are counted in blocks: recent = the r blocks ending
    at the diagonal, window = the w blocks just before those, sink = the first
    s blocks;
  * the row normalisation uses epsilon = 0; ties at the threshold are kept
    (Score >= thresh);
  * |B_J| is the actual token count of block J (the last block may be short);
  * a query row that sees no key at all gets O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math

import numpy as np


def n_blocks(L: int, B: int) -> int:
    return (L + B - 1) // B


def pool_means(x: np.ndarray, B: int) -> np.ndarray:
    """Mean-pooled block vectors, k_bar_J = (1/|B_J|) sum_{i in B_J} k_i
    ([V2] Sec. 3.1 first paragraph; [V1] method steps).  Also used for the
    pooled values v_bar_J of the correction ([V2] Sec. 3.2, Fig. 6 text:
    "pooled K/V means").  x: [L, H, d] float64 -> [N, H, d]."""
    L = x.shape[0]
    N = n_blocks(L, B)
    out = np.empty((N,) + x.shape[1:], dtype=np.float64)
    for J in range(N):
        out[J] = x[J * B:min((J + 1) * B, L)].astype(np.float64).mean(axis=0)
    return out


def tile_query_rows(q: np.ndarray, h: int, g: int, B: int, I: int, q_off: int = 0):
    """Rows of selection tile I for KV head h: the query positions inside
    block I, max(I*B, q_off) .. min((I+1)*B, L)-1, times the g query heads
    h*g .. h*g+g-1 of the group (PackGQA row order: position-major,
    head-minor, [V2] PackGQA paragraph).  q: [L - q_off, Hq, d] holds the
    queries of positions q_off .. L-1, where L is the key count: a whole
    prompt has q_off = 0, a chunk of a chunked prefill ([V2] integration
    paragraph) the position of its first query.
    Returns (positions [rows], head index [rows], vectors [rows, d])."""
    L = q.shape[0] + q_off
    pos = np.arange(max(I * B, q_off), min((I + 1) * B, L))
    heads = np.arange(h * g, (h + 1) * g)
    rows = q[pos - q_off][:, heads, :].reshape(-1, q.shape[2]).astype(np.float64)
    return np.repeat(pos, g), np.tile(heads, len(pos)), rows


def block_scores_row(q_rows: np.ndarray, kbar_h: np.ndarray, I: int, scale: float) -> np.ndarray:
    """Score_{I,J} for J = 0..I ([V1] method steps; [V2] Sec. 3.1).

    s_{r,J} = scale * q_r . k_bar_J                 (block-causal J <= I)
    M_I     = max over rows r and J <= I of s_{r,J}
    S'_{IJ} = sum_r exp(s_{r,J} - M_I)
    Score   = S'_{IJ} / sum_K S'_{IK}               (epsilon = 0)

    [V1] writes S'_{IJ} = S_{IJ} exp(m_{IJ} - M_I) with the per-block max
    m_{IJ} and S_{IJ} = sum_r exp(s_{rJ} - m_{IJ}); that product is the same
    number as the sum above.
    """
    s = scale * (q_rows @ kbar_h[:I + 1].T)  # [rows, I+1]
    M = s.max()
    Sp = np.exp(s - M).sum(axis=0)
    return Sp / Sp.sum()


def forced_blocks(I: int, sink: int, window: int, recent: int):
    """Sink, sliding-window and recent blocks of tile I, causal (J <= I)
    ([V2] Sec. 3.1, threshold paragraph; sizes counted in blocks)."""
    sink_set = set(range(0, min(sink, I + 1)))
    recent_set = set(range(max(0, I - recent + 1), I + 1))
    window_set = set(range(max(0, I - recent - window + 1), max(0, I - recent + 1)))
    return sink_set | window_set | recent_set


def select_row(score: np.ndarray, I: int, alpha: float, sink: int, window: int, recent: int):
    """Max-based dynamic threshold ([V1] core method: thresh_I = alpha * max_{J<=I}
    Score_{I,J}; [V2] Sec. 3.1: keep Score >= thresh plus the forced blocks).
    Returns (ascending selected list, thresh)."""
    thresh = alpha * score.max()
    kept = {int(J) for J in np.nonzero(score >= thresh)[0]}
    sel = sorted(kept | forced_blocks(I, sink, window, recent))
    return sel, thresh


def todo_row(sel, I: int, correction: bool):
    """Blocks corrected with their pooled means: valid & ~selected, where valid
    are the blocks fully visible to every query of tile I, i.e. J <= I-1
    ([V2] Sec. 3.2, Fig. 3 green path and the todo bitmask)."""
    if not correction:
        return []
    s = set(sel)
    return [J for J in range(I) if J not in s]


def attend_rows(pos, q_rows, k_h, v_h, kbar_h, vbar_h, sel, todo, B: int, scale: float,
                p_scale: float = 1.0, return_state: bool = False):
    """Block-sparse causal attention with mean correction for a set of query
    rows of one tile ([V2] Sec. 3.1 last sentence, Sec. 3.2).

    Exact terms    e_j = scale * q . k_j for the tokens j of the selected
                   blocks with j <= i (token-level causal mask).
    Correction     c_J = scale * q . k_bar_J + ln|B_J| for J in todo: one
                   pooled vector stands for |B_J| tokens in numerator and
                   denominator ([V2] Sec. 3.2, Fig. 3 paragraph).
    With m = max of all terms:
      O   = (sum_j e^{e_j-m} v_j + sum_J e^{c_J-m} v_bar_J) / l,
      l   = sum_j e^{e_j-m} + sum_J e^{c_J-m},
      LSE = m + ln l.
    p_scale multiplies every probability before it is summed (the FP8 path
    scales probabilities by 2^8, [V2] FP8 paragraph); LSE is reported with
    ln(p_scale) removed, as that paragraph says it is recovered at finalize.
    """
    L = k_h.shape[0]
    pos = np.asarray(pos)
    keys = np.concatenate([np.arange(J * B, min((J + 1) * B, L)) for J in sel]) \
        if len(sel) else np.zeros(0, dtype=np.int64)
    e = scale * (q_rows @ k_h[keys].astype(np.float64).T)
    e = np.where(keys[None, :] <= pos[:, None], e, -np.inf)
    todo = list(todo)
    if todo:
        sizes = np.array([min((J + 1) * B, L) - J * B for J in todo], dtype=np.float64)
        c = scale * (q_rows @ kbar_h[todo].T) + np.log(sizes)[None, :]
        vals = np.concatenate([v_h[keys].astype(np.float64), vbar_h[todo]], axis=0)
    else:
        c = np.zeros((len(pos), 0))
        vals = v_h[keys].astype(np.float64)
    t = np.concatenate([e, c], axis=1)
    m = t.max(axis=1) if t.shape[1] else np.full(len(pos), -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(t - m_safe[:, None]) * p_scale
    ell = w.sum(axis=1)
    num = w @ vals
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(empty[:, None], 0.0, num / np.where(empty, 1.0, ell)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, ell)) - math.log(p_scale))
    if return_state:
        return O, lse, m, ell / p_scale
    return O, lse


def merge_partials(O1, l1, m1, O2, l2, m2):
    """Online-softmax merge of two partial results over disjoint key sets
    ([PRR] Sec. 4.3, Eq. 6): l is used as a plain sum of exponentials and O as
    the normalised partial output."""
    m = np.maximum(m1, m2)
    a1 = np.exp(m1 - m) * l1
    a2 = np.exp(m2 - m) * l2
    ell = a1 + a2
    O = (a1 / ell)[:, None] * O1 + (a2 / ell)[:, None] * O2
    return O, ell, m


def dense_causal_reference(q, k, v, scale: float):
    """Textbook causal softmax attention of one request (an explicit L x L
    masked score matrix per head), for pins only.  q [L, Hq, d], k/v [L, Hkv, d]."""
    L, Hq, d = q.shape
    g = Hq // k.shape[1]
    O = np.empty((L, Hq, d))
    lse = np.empty((Hq, L))
    mask = np.tril(np.ones((L, L), dtype=bool))
    for hq in range(Hq):
        h = hq // g
        S = scale * (q[:, hq, :].astype(np.float64) @ k[:, h, :].astype(np.float64).T)
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        lse[hq] = m[:, 0] + np.log(P.sum(axis=1))
        O[:, hq, :] = (P / P.sum(axis=1, keepdims=True)) @ v[:, h, :].astype(np.float64)
    return O, lse


def request_oracle(q, k, v, B: int, scale: float, alpha: float, sink: int, window: int,
                   recent: int, correction: bool, tiles=None, heads=None):
    """Whole pipeline for one request, the steps in the pages' order.

    q [Lq, Hq, d], k/v [L, Hkv, d] as float64 (already dequantised); the
    queries are the last Lq positions (Lq = L for a whole prompt, fewer for a
    chunk of a chunked prefill, whose index is re-run over its own tiles).
    `tiles` / `heads` restrict the work to some (KV head, tile) pairs; by
    default every pair is computed.

    Returns a dict with kbar/vbar [N, Hkv, d] and, per (h, I): score row,
    thresh, sel, todo, and the tile's output rows (positions, query heads,
    O [rows, d], LSE [rows]).
    """
    Lq, Hq, d = q.shape
    L = k.shape[0]
    q_off = L - Lq
    Hkv = k.shape[1]
    g = Hq // Hkv
    N = n_blocks(L, B)
    I0 = q_off // B if Lq else N  # first tile that holds a query
    kbar = pool_means(k, B)
    vbar = pool_means(v, B)
    out = {"kbar": kbar, "vbar": vbar, "tiles": {}}
    heads = range(Hkv) if heads is None else heads
    for h in heads:
        kh = k[:, h, :].astype(np.float64)
        vh = v[:, h, :].astype(np.float64)
        for I in (range(I0, N) if tiles is None else tiles):
            pos, hqs, rows = tile_query_rows(q, h, g, B, I, q_off)
            score = block_scores_row(rows, kbar[:, h, :], I, scale)
            sel, thresh = select_row(score, I, alpha, sink, window, recent)
            todo = todo_row(sel, I, correction)
            O, lse = attend_rows(pos, rows, kh, vh, kbar[:, h, :], vbar[:, h, :], sel, todo, B,
                                 scale)
            out["tiles"][(h, I)] = dict(score=score, thresh=thresh, sel=sel, todo=todo,
                                        pos=pos, heads=hqs, O=O, lse=lse)
    return out


def packgqa_rows(L: int, g: int):
    """PackGQA view of one KV group ([V2] PackGQA paragraph): packed row r maps
    to position r div g and group head r mod g.  Returns [(pos, head)] for
    r = 0 .. g*L-1."""
    return [(r // g, r % g) for r in range(g * L)]


def wasted_row_fraction(L: int, g: int, kBlockM: int, packed: bool) -> float:
    """Fraction of M-tile rows left empty, counted by enumerating tiles: per
    head under the naive mapping (L rows per head), once per group under
    PackGQA (g*L packed rows)."""
    rows = g * L if packed else L
    tiles = -(-rows // kBlockM)
    return (tiles * kBlockM - rows) / (tiles * kBlockM)
