"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test is chosen so that a plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong mask) fails at
least one of them.  All CPU-only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import TINY_F32, generate_f32

HERE = os.path.dirname(os.path.abspath(__file__))


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    if x.startswith("ln"):
        return math.log(float(Fraction(x[2:])))
    return float(Fraction(x))


def _arr(a):
    return np.array([[_num(e) for e in row] if isinstance(row, list) else _num(row) for row in a],
                    dtype=np.float64)


# ---------------------------------------------------------------- golden fixture

@pytest.fixture(scope="module")
def golden():
    with open(os.path.join(HERE, "golden", "closed_form_tiny.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("correction", [True, False])
def test_golden_closed_form(golden, correction):
    g = golden
    k = _arr(g["k"])[:, None, :]
    v = _arr(g["v"])[:, None, :]
    q = _arr(g["q"])[:, None, :]
    res = oracle.request_oracle(q, k, v, g["B"], g["scale"], g["alpha"], g["sink"], g["window"],
                                g["recent"], correction)
    ex = g["expected"]
    np.testing.assert_allclose(res["kbar"][:, 0], _arr(ex["kbar"]), atol=1e-15)
    np.testing.assert_allclose(res["vbar"][:, 0], _arr(ex["vbar"]), atol=1e-15)
    O = np.zeros((6, 2))
    lse = np.zeros(6)
    for I in range(3):
        t = res["tiles"][(0, I)]
        np.testing.assert_allclose(t["score"], _arr(ex["score"][str(I)]), rtol=1e-14)
        assert t["thresh"] == pytest.approx(_num(ex["thresh"][str(I)]), rel=1e-14)
        assert t["sel"] == ex["sel"][str(I)]
        assert t["todo"] == (ex["todo_corrected"][str(I)] if correction else [])
        O[t["pos"]] = t["O"]
        lse[t["pos"]] = t["lse"]
    key = "corrected" if correction else "dropped"
    np.testing.assert_allclose(O, _arr(ex["O_" + key]), atol=1e-14)
    np.testing.assert_allclose(lse, _arr(ex["lse_" + key]), atol=1e-14)


# ---------------------------------------------------------------- textbook attention

def _bruteforce_dense(q, k, v, scale):
    """Causal softmax attention written out with explicit loops (tiny sizes)."""
    L, Hq, d = q.shape
    g = Hq // k.shape[1]
    O = np.zeros((L, Hq, d))
    lse = np.zeros((Hq, L))
    for hq in range(Hq):
        h = hq // g
        for i in range(L):
            logits = [scale * float(np.dot(q[i, hq], k[j, h])) for j in range(i + 1)]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            s = sum(w)
            lse[hq, i] = m + math.log(s)
            for j in range(i + 1):
                O[i, hq] += (w[j] / s) * v[j, h]
    return O, lse


def _assemble(res, L, Hq, d):
    O = np.full((L, Hq, d), np.nan)
    lse = np.full((Hq, L), np.nan)
    for t in res["tiles"].values():
        O[t["pos"], t["heads"]] = t["O"]
        lse[t["heads"], t["pos"]] = t["lse"]
    return O, lse


@pytest.mark.parametrize("correction", [True, False])
@pytest.mark.parametrize("L,B,Hq,Hkv", [(37, 8, 4, 2), (64, 16, 2, 2), (23, 32, 3, 1)])
def test_alpha_zero_equals_dense_bruteforce(L, B, Hq, Hkv, correction):
    rng = np.random.default_rng(L * 100 + B)
    d = 8
    q = rng.standard_normal((L, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    scale = 1 / math.sqrt(d)
    res = oracle.request_oracle(q, k, v, B, scale, 0.0, 0, 0, 0, correction)
    for t in res["tiles"].values():
        assert t["todo"] == []
    O, lse = _assemble(res, L, Hq, d)
    Ob, lseb = _bruteforce_dense(q, k, v, scale)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, atol=1e-12)
    Od, lsed = oracle.dense_causal_reference(q, k, v, scale)
    np.testing.assert_allclose(Od, Ob, atol=1e-12)
    np.testing.assert_allclose(lsed, lseb, atol=1e-12)


def test_identical_keys_give_uniform_average():
    """All keys equal: every visible key gets the same weight, so O_i is the
    plain mean of v_0..v_i and LSE_i = s + ln(i+1), whatever alpha is."""
    rng = np.random.default_rng(3)
    L, B, d = 40, 8, 4
    kvec = rng.standard_normal(d)
    k = np.tile(kvec, (L, 1))[:, None, :]
    v = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((L, 1, d))
    res = oracle.request_oracle(q, k, v, B, 0.5, 0.3, 1, 1, 1, True)
    O, lse = _assemble(res, L, 1, d)
    for i in range(L):
        np.testing.assert_allclose(O[i, 0], v[:i + 1, 0].mean(axis=0), atol=1e-13)
        assert lse[0, i] == pytest.approx(0.5 * q[i, 0] @ kvec + math.log(i + 1), abs=1e-12)


# ---------------------------------------------------------------- mean correction

def _constant_key_problem(seed, L=96, B=8, Hq=2, Hkv=1, d=6):
    rng = np.random.default_rng(seed)
    N = -(-L // B)
    cent = 1.5 * rng.standard_normal((N, Hkv, d))
    k = np.repeat(cent, B, axis=0)[:L]  # keys constant inside every block
    v = rng.standard_normal((L, Hkv, d))
    q = rng.standard_normal((L, Hq, d)) + 2.0 * cent[rng.integers(0, N, L)][:, :, :].repeat(Hq // Hkv, 1)
    return q, k, v, B


def test_correction_exact_for_constant_key_blocks():
    """With delta_i = 0 inside every block the mass surrogate |B_J| e^{s_bar}
    equals the block mass and the covariance term vanishes, so corrected
    sparse attention equals dense attention for any alpha (FlashPrefill V2,
    Sec. 3.2, Eq. 6 / Eq. 8 and bound (ii)); dropping instead does not."""
    q, k, v, B = _constant_key_problem(11)
    L, Hq, d = q.shape
    scale = 1 / math.sqrt(d)
    Od, lsed = oracle.dense_causal_reference(q, k, v, scale)
    res = oracle.request_oracle(q, k, v, B, scale, 0.5, 1, 0, 1, True)
    assert sum(len(t["todo"]) for t in res["tiles"].values()) > 0
    O, lse = _assemble(res, L, Hq, d)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)
    res2 = oracle.request_oracle(q, k, v, B, scale, 0.5, 1, 0, 1, False)
    O2, _ = _assemble(res2, L, Hq, d)
    assert np.abs(O2 - Od).max() > 1e-3


def test_correction_uses_actual_block_size():
    """A short final block contributes ln|B_J| with its own token count.  The
    short block is only ever corrected when it is fully visible, which
    happens for none of the tiles; so check the log-size term on the
    full blocks against a hand-built sum."""
    rng = np.random.default_rng(5)
    L, B, d = 20, 8, 3
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((L, 1, d))
    kbar = oracle.pool_means(k, B)[:, 0]
    vbar = oracle.pool_means(v, B)[:, 0]
    pos = np.array([19])
    O, lse = oracle.attend_rows(pos, q[19:20, 0], k[:, 0], v[:, 0], kbar, vbar, [2], [0, 1], B, 1.0)
    terms = [(q[19, 0] @ k[j, 0], v[j, 0]) for j in range(16, 20)]
    terms += [(q[19, 0] @ kbar[J] + math.log(8), vbar[J]) for J in (0, 1)]
    m = max(t for t, _ in terms)
    ell = sum(math.exp(t - m) for t, _ in terms)
    num = sum(math.exp(t - m) * vv for t, vv in terms)
    np.testing.assert_allclose(O[0], num / ell, atol=1e-14)
    assert lse[0] == pytest.approx(m + math.log(ell), abs=1e-14)
    np.testing.assert_allclose(kbar[2], k[16:20, 0].mean(axis=0), atol=1e-15)


def test_drop_identity():
    """Dropping block J shifts the output by exactly (w_J / D)(mu_J - O_drop),
    with w_J the block mass, D the total mass and mu_J the block's
    mass-weighted value mean (FlashPrefill V2, Sec. 3.2, bound (iii))."""
    rng = np.random.default_rng(8)
    L, B, d = 64, 8, 5
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((L, 1, d))
    kbar = oracle.pool_means(k, B)[:, 0]
    vbar = oracle.pool_means(v, B)[:, 0]
    i = 60
    I = i // B
    everything = list(range(I + 1))
    for J in range(I):
        O_full, _ = oracle.attend_rows([i], q[i:i + 1, 0], k[:, 0], v[:, 0], kbar, vbar,
                                       everything, [], B, 1.0)
        kept = [x for x in everything if x != J]
        O_drop, _ = oracle.attend_rows([i], q[i:i + 1, 0], k[:, 0], v[:, 0], kbar, vbar,
                                       kept, [], B, 1.0)
        s = np.array([q[i, 0] @ k[j, 0] for j in range(i + 1)])
        w_all = np.exp(s)
        D = w_all.sum()
        blk = slice(J * B, (J + 1) * B)
        wJ = w_all[blk].sum()
        muJ = (w_all[blk, None] * v[blk, 0]).sum(axis=0) / wJ
        np.testing.assert_allclose(O_full[0] - O_drop[0], (wJ / D) * (muJ - O_drop[0]), atol=1e-13)


def test_merge_recurrence_equals_unsplit():
    """Attention over A u B equals the online-softmax merge of the partials
    over A and over B (PRR review, Sec. 4.3, Eq. 6)."""
    rng = np.random.default_rng(9)
    L, B, d = 128, 16, 6
    k = rng.standard_normal((L, 1, d)) * 2
    v = rng.standard_normal((L, 1, d))
    q = rng.standard_normal((16, d))
    kbar = oracle.pool_means(k, B)[:, 0]
    vbar = oracle.pool_means(v, B)[:, 0]
    pos = np.arange(112, 128)
    sel_a, todo_a = [0, 7], [2, 3]
    sel_b, todo_b = [4, 5], [1, 6]
    Oa, _, ma, la = oracle.attend_rows(pos, q, k[:, 0], v[:, 0], kbar, vbar, sel_a, todo_a, B, 0.7,
                                       return_state=True)
    Ob, _, mb, lb = oracle.attend_rows(pos, q, k[:, 0], v[:, 0], kbar, vbar, sel_b, todo_b, B, 0.7,
                                       return_state=True)
    Om, lm, mm = oracle.merge_partials(Oa, la, ma, Ob, lb, mb)
    Ou, lseu = oracle.attend_rows(pos, q, k[:, 0], v[:, 0], kbar, vbar, sel_a + sel_b,
                                  todo_a + todo_b, B, 0.7)
    np.testing.assert_allclose(Om, Ou, atol=1e-13)
    np.testing.assert_allclose(mm + np.log(lm), lseu, atol=1e-13)


def test_fp8_probability_offset_cancels():
    """Scaling every probability by 2^8 leaves O unchanged and is removed from
    the LSE at finalize (FlashPrefill V2, FP8 paragraph)."""
    rng = np.random.default_rng(10)
    L, B, d = 64, 16, 4
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    q = rng.standard_normal((16, d))
    kbar = oracle.pool_means(k[:, None], B)[:, 0]
    vbar = oracle.pool_means(v[:, None], B)[:, 0]
    pos = np.arange(48, 64)
    O1, l1 = oracle.attend_rows(pos, q, k, v, kbar, vbar, [1, 3], [0, 2], B, 0.5)
    O2, l2 = oracle.attend_rows(pos, q, k, v, kbar, vbar, [1, 3], [0, 2], B, 0.5, p_scale=256.0)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


# ---------------------------------------------------------------- pooling / scores

def test_amgm_lower_bound_on_planted_inputs():
    """exp(q . k_bar_J) <= mean_i exp(q . k_i) for every block (AM-GM,
    FlashPrefill V2 Sec. 3.1), with equality for a constant block."""
    q, k, v = generate_f32(TINY_F32.replace(seqlens=(512,)), 0)
    B = 64
    kbar = oracle.pool_means(k.astype(np.float64), B)[:, 0]
    rng = np.random.default_rng(0)
    qs = q[rng.integers(0, 512, 64), 0].astype(np.float64) / 8.0
    for J in range(kbar.shape[0]):
        blk = k[J * B:(J + 1) * B, 0].astype(np.float64)
        lhs = np.exp(qs @ kbar[J])
        rhs = np.exp(qs @ blk.T).mean(axis=1)
        assert np.all(lhs <= rhs * (1 + 1e-12))
        assert np.all(lhs < rhs)  # strict: keys vary inside the block
    const = np.tile(k[:1, 0], (B, 1)).astype(np.float64)
    cbar = oracle.pool_means(const[:, None], B)[0, 0]
    np.testing.assert_allclose(np.exp(qs @ cbar), np.exp(qs @ const.T).mean(axis=1), rtol=1e-12)


def test_pool_means_partial_and_constant():
    x = np.arange(10 * 2 * 3, dtype=np.float64).reshape(10, 2, 3)
    m = oracle.pool_means(x, 4)
    assert m.shape == (3, 2, 3)
    np.testing.assert_allclose(m[0], x[0:4].sum(axis=0) / 4)
    np.testing.assert_allclose(m[2], (x[8] + x[9]) / 2)


def test_score_row_matches_v1_two_stage_reduction():
    """The V1 page computes per-block m_IJ and S_IJ and then rescales by
    M_I; with one global max the same numbers come out."""
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((24, 8)) * 3
    kbar = rng.standard_normal((7, 8))
    score = oracle.block_scores_row(rows, kbar, 6, 0.4)
    s = 0.4 * rows @ kbar.T
    m = s.max(axis=0)
    S = np.exp(s - m).sum(axis=0)
    M = m.max()
    Sp = S * np.exp(m - M)
    np.testing.assert_allclose(score, Sp / Sp.sum(), rtol=1e-13)
    assert score.sum() == pytest.approx(1.0, abs=1e-14)


def test_score_block_causal_and_row_order():
    """Scores only look at J <= I and see every row of the tile: changing a
    key block beyond I must not change row I; changing a query of another
    tile must not either; changing one query of the tile must."""
    rng = np.random.default_rng(12)
    L, B, Hq, Hkv, d = 64, 8, 4, 2, 4
    q = rng.standard_normal((L, Hq, d))
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    base = oracle.request_oracle(q, k, v, B, 0.5, 0.1, 0, 0, 1, True, tiles=[3], heads=[1])
    k2 = k.copy()
    k2[4 * B:, 1] += 5.0
    q2 = q.copy()
    q2[5 * B, 2:4] += 5.0
    alt = oracle.request_oracle(q2, k2, v, B, 0.5, 0.1, 0, 0, 1, True, tiles=[3], heads=[1])
    np.testing.assert_allclose(alt["tiles"][(1, 3)]["score"], base["tiles"][(1, 3)]["score"])
    q3 = q.copy()
    q3[3 * B + 2, 3] += 1.0  # query head 3 belongs to KV head 1
    alt3 = oracle.request_oracle(q3, k, v, B, 0.5, 0.1, 0, 0, 1, True, tiles=[3], heads=[1])
    assert np.abs(alt3["tiles"][(1, 3)]["score"] - base["tiles"][(1, 3)]["score"]).max() > 1e-6
    q4 = q.copy()
    q4[3 * B + 2, 0] += 1.0  # query head 0 belongs to KV head 0
    alt4 = oracle.request_oracle(q4, k, v, B, 0.5, 0.1, 0, 0, 1, True, tiles=[3], heads=[1])
    np.testing.assert_allclose(alt4["tiles"][(1, 3)]["score"], base["tiles"][(1, 3)]["score"])


# ---------------------------------------------------------------- selection

def test_forced_blocks_reading():
    # sink 1, window 2, recent 1 force {0, I-2, I-1, I}
    assert oracle.forced_blocks(10, 1, 2, 1) == {0, 8, 9, 10}
    assert oracle.forced_blocks(2, 1, 2, 1) == {0, 1, 2}
    assert oracle.forced_blocks(0, 1, 2, 1) == {0}
    assert oracle.forced_blocks(10, 2, 0, 3) == {0, 1, 8, 9, 10}
    assert oracle.forced_blocks(10, 0, 3, 0) == {8, 9, 10}
    assert oracle.forced_blocks(5, 0, 0, 0) == set()


@pytest.mark.parametrize("forced_args", [(1, 2, 1), (0, 0, 0)])
def test_selection_invariants_on_planted_inputs(forced_args):
    w = TINY_F32
    q, k, v = (a.astype(np.float64) for a in generate_f32(w, 1))
    alphas = [0.4, 0.2, 0.05, 0.01, 0.0]
    prev = None
    diag_dropped = 0
    for a in alphas:
        res = oracle.request_oracle(q, k, v, w.block, w.scale, a, *forced_args, True, heads=[0])
        sels = {}
        for (h, I), t in res["tiles"].items():
            sel = set(t["sel"])
            diag_dropped += I not in sel
            forced = oracle.forced_blocks(I, *forced_args)
            assert forced <= sel <= set(range(I + 1))
            assert t["sel"] == sorted(sel)
            for J in range(I + 1):
                if J not in forced:
                    assert (t["score"][J] >= t["thresh"]) == (J in sel)
            assert set(t["todo"]) == set(range(I)) - sel
            if a == 0.0:
                assert sel == set(range(I + 1))
            sels[I] = sel
        if prev is not None:  # smaller alpha keeps a superset
            for I in sels:
                assert prev[I] <= sels[I]
        prev = sels
    if forced_args == (0, 0, 0):
        # the diagonal block is never fully visible, so a dropped diagonal
        # is neither attended nor corrected
        assert diag_dropped > 0


def test_alpha_zero_keeps_underflowed_blocks():
    score = np.array([0.0, 1.0, 0.0])
    sel, thresh = oracle.select_row(score, 2, 0.0, 0, 0, 0)
    assert sel == [0, 1, 2] and thresh == 0.0
    sel, _ = oracle.select_row(score, 2, 1e-300, 0, 0, 0)
    assert sel == [1]


# ---------------------------------------------------------------- PackGQA, fp8

@pytest.mark.parametrize("L,g,M", [(1, 4, 128), (1, 8, 128), (100, 4, 128), (1000, 8, 128),
                                   (16384, 4, 128), (3, 32, 64)])
def test_packgqa_wasted_rows_formula(L, g, M):
    """Printed wasted-row fractions of the naive and packed mappings
    (FlashPrefill V2, PackGQA paragraph), against tile enumeration."""
    naive = (math.ceil(L / M) * M - L) / (math.ceil(L / M) * M)
    packed = (math.ceil(g * L / M) * M - g * L) / (math.ceil(g * L / M) * M)
    assert oracle.wasted_row_fraction(L, g, M, False) == pytest.approx(naive)
    assert oracle.wasted_row_fraction(L, g, M, True) == pytest.approx(packed)
    rows = oracle.packgqa_rows(L, g)
    assert len(rows) == g * L and len(set(rows)) == g * L
    if L * g <= M:  # decode-like: one packed tile instead of g naive tiles
        assert math.ceil(g * L / M) == 1


def test_tile_rows_follow_packgqa_order():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((20, 8, 3))
    pos, heads, rows = oracle.tile_query_rows(q, 1, 4, 8, 1)
    packed = oracle.packgqa_rows(8, 4)
    for r, (p, hh) in enumerate(packed):
        assert pos[r] == 8 + p and heads[r] == 4 + hh
        np.testing.assert_array_equal(rows[r], q[8 + p, 4 + hh])


def test_fp8_decoder_matches_torch():
    import torch
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    ours = oracle.decode_e4m3fn(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and ours[1] == 2.0 ** -9


# ---------------------------------------------------------------- online fp8 quantisation

def test_e4m3_encoder_round_trips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode_e4m3fn(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(oracle.encode_e4m3fn(vals[ok]), codes[ok])


def test_e4m3_encoder_rounds_to_nearest_even_and_saturates():
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A: midpoints go to the even code
    assert oracle.encode_e4m3fn([1.0625, 1.1875])[0] == 0x38
    assert oracle.encode_e4m3fn([1.1875])[0] == 0x3A
    assert oracle.encode_e4m3fn([1.0624, 1.0626]).tolist() == [0x38, 0x39]
    # the smallest subnormal is 2^-9 (0x01); half of it ties to zero, a bit more rounds up
    assert oracle.encode_e4m3fn([2.0 ** -10, 2.0 ** -10 * 1.01]).tolist() == [0x00, 0x01]
    # above 448 (0x7E) saturates, with the sign kept
    assert oracle.encode_e4m3fn([464.0, 1e30, -1e30]).tolist() == [0x7E, 0x7E, 0xFE]


def test_e4m3_encoder_matches_torch_cast():
    import torch
    x = np.random.default_rng(3).standard_normal(20000).astype(np.float32) * 60
    ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3fn(x), ref)


def test_quantize_per_tensor_scale_and_error():
    x = np.random.default_rng(4).standard_normal(5000).astype(np.float32) * 3
    codes, scale = oracle.quantize_per_tensor(x)
    assert scale == np.float32(np.float32(np.abs(x).max()) / np.float32(448))
    # the absmax element lands on 448 exactly
    i = int(np.argmax(np.abs(x)))
    assert abs(oracle.decode_e4m3fn(codes[i])) == 448.0
    # every other element within half an e4m3 step (relative 2^-4, or the subnormal step)
    back = oracle.decode_e4m3fn(codes) * float(scale)
    step = np.maximum(np.abs(x) * 2.0 ** -3, 2.0 ** -9 * float(scale))
    assert np.all(np.abs(back - x) <= 0.5 * step + 1e-12)
    z_codes, z_scale = oracle.quantize_per_tensor(np.zeros(7, np.float32))
    assert z_scale == 1.0 and not z_codes.any()


# ---------------------------------------------------------------- chunked prefill

def _planted(L, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, Hkv, d))
    v = rng.standard_normal((L, Hkv, d))
    q = rng.standard_normal((L, Hq, d)) + np.repeat(k, Hq // Hkv, axis=1) * 1.5
    return q, k, v


@pytest.mark.parametrize("alpha,correction", [(0.2, True), (0.05, False), (0.0, True)])
def test_block_aligned_chunk_reproduces_the_whole_prompt_tiles(alpha, correction):
    # a chunk that starts on a block boundary has exactly the whole prompt's
    # tiles I >= i0 (same rows), so scores, selection and outputs agree
    B, L, off = 16, 150, 64
    q, k, v = _planted(L, 4, 2, 8, 5)
    args = (B, 1 / np.sqrt(8), alpha, 1, 1, 1, correction)
    whole = oracle.request_oracle(q, k, v, *args)
    chunk = oracle.request_oracle(q[off:], k, v, *args)
    assert set(chunk["tiles"]) == {(h, I) for h in range(2) for I in range(off // B, 10)}
    for key, t in chunk["tiles"].items():
        w = whole["tiles"][key]
        assert t["sel"] == w["sel"] and t["todo"] == w["todo"]
        assert np.array_equal(t["pos"], w["pos"]) and np.array_equal(t["score"], w["score"])
        assert np.array_equal(t["O"], w["O"]) and np.array_equal(t["lse"], w["lse"])


def test_unaligned_chunk_dense_rows_are_textbook_attention():
    # alpha = 0 without correction: every query of a chunk (first tile cut
    # mid-block) attends to all keys up to its position
    B, L, off = 16, 100, 37
    q, k, v = _planted(L, 4, 2, 8, 6)
    scale = 1 / np.sqrt(8)
    chunk = oracle.request_oracle(q[off:], k, v, B, scale, 0.0, 1, 1, 1, False)
    Od, lsed = oracle.dense_causal_reference(q, k, v, scale)
    first = chunk["tiles"][(0, off // B)]
    assert first["pos"].min() == off and len(set(first["pos"])) == (off // B + 1) * B - off
    for t in chunk["tiles"].values():
        assert np.allclose(t["O"], Od[t["pos"], t["heads"]], atol=1e-12)
        assert np.allclose(t["lse"], lsed[t["heads"], t["pos"]], atol=1e-12)


# ---------------------------------------------------------------- FP8 attention arithmetic

def _fp8_golden():
    with open(os.path.join(HERE, "golden", "fp8_walk_tiny.json")) as f:
        return json.load(f)


def test_fp8_walk_golden_running_max():
    """The e4m3 probabilities are rounded against the running maximum of a
    backwards walk: hand-derived values (tests/golden/fp8_walk_tiny.json)."""
    g = _fp8_golden()["walk"]
    L, B = g["L"], g["B"]
    k = np.zeros((L, 2))
    k[:, 0] = -1000.0
    for j, s in g["s"].items():
        k[int(j), 0] = _num(s)
    v = np.zeros((L, 2))
    for j, val in g["v"].items():
        v[int(j)] = val
    kbar = oracle.pool_means(k[:, None], B)[:, 0]
    vbar = oracle.pool_means(v[:, None], B)[:, 0]
    q = np.array([[1.0, 0.0]])
    O, lse = oracle.attend_rows_fp8([g["pos"]], q, k, v, g["sel"], g["todo"], B, 1.0, 1.0, 1.0)
    np.testing.assert_allclose(O[0], [_num(x) for x in g["expected_O"]], atol=1e-13)
    np.testing.assert_allclose(lse[0], _num(g["expected_lse"]), atol=1e-13)
    # the exact arithmetic differs (LSE ln 2.8): the rounding is really applied
    _, lse_x = oracle.attend_rows([g["pos"]], q, k, v, kbar, vbar, g["sel"], g["todo"], B, 1.0)
    assert abs(lse_x[0] - math.log(2.8)) < 1e-12 and abs(lse[0] - lse_x[0]) > 1e-3


def test_fp8_walk_golden_quantised_pooled_statistics():
    g = _fp8_golden()["correction"]
    L, B = g["L"], g["B"]
    ck = float(g["k_scale"])
    sc = math.log(2) / 4  # softmax scale
    k = np.zeros((L, 2))
    k[g["pos"] + 1:, 0] = 1e3  # keys after the row are masked anyway
    v = np.zeros((L, 2))
    v[128] = g["v128"]
    for J in (0, 1):
        keys, vals = _arr(g[f"block{J}_keys"]), _arr(g[f"block{J}_values"])
        for half in (0, 1):
            rows = slice(J * B + 32 * half, J * B + 32 * half + 32)
            k[rows] = keys[half] * ck
            v[rows] = vals[half]
    q = np.array([[1.0, 0.0]])
    O, lse = oracle.attend_rows_fp8([g["pos"]], q, k, v, g["sel"], g["todo"], B, sc, ck, 1.0)
    np.testing.assert_allclose(O[0], [_num(x) for x in g["expected_O"]], atol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(7 / 4), atol=1e-12)
    # unrounded pooled statistics would give other weights
    kbar = oracle.pool_means(k[:, None], B)[:, 0]
    vbar = oracle.pool_means(v[:, None], B)[:, 0]
    O_x, _ = oracle.attend_rows([g["pos"]], q, k, v, kbar, vbar, g["sel"], g["todo"], B, sc)
    assert np.abs(O_x[0] - O[0]).max() > 1e-2


def test_fp8_pooled_code_means_are_exact():
    """Block means of the codes are recovered exactly from code * scale, so a
    mean that sits on an e4m3 midpoint is a true tie (rounded to even)."""
    rng = np.random.default_rng(3)
    codes = oracle.decode_e4m3fn(rng.integers(0, 0x7E, size=(256, 4)).astype(np.uint8))
    scale = 0.0123456789
    means = oracle.pooled_code_means(codes * scale, scale, 64)
    exact = np.stack([codes[i * 64:(i + 1) * 64].mean(axis=0) for i in range(4)])
    np.testing.assert_array_equal(means, exact)
    # a block of 32 codes 28 and 32 codes 30: mean 29, the midpoint of 28 and 30
    block = np.array([[28.0]] * 32 + [[30.0]] * 32)
    m = oracle.pooled_code_means(block * 0.37, 0.37, 64)
    assert m[0, 0] == 29.0 and oracle.e4m3_round(m)[0, 0] == 28.0


def test_fp8_near_tie_flip_changes_one_rounding():
    """A probability within the tie band is reported, and forcing its other
    rounding changes the result by that one weight (the golden walk: key 65
    has P = 76.8, not near a midpoint; with a wide band it is reported)."""
    g = _fp8_golden()["walk"]
    L, B = g["L"], g["B"]
    k = np.zeros((L, 2))
    k[:, 0] = -1000.0
    for j, s in g["s"].items():
        k[int(j), 0] = _num(s)
    v = np.zeros((L, 2))
    for j, val in g["v"].items():
        v[int(j)] = val
    q = np.array([[1.0, 0.0]])
    O0, l0, near = oracle.attend_rows_fp8([g["pos"]], q, k, v, g["sel"], g["todo"], B, 1.0, 1.0,
                                          1.0, tie_band=0.05)
    assert 65 in near[0]  # 76.8 is 0.8 from the midpoint 76 (1%)
    O1, l1 = oracle.attend_rows_fp8([g["pos"]], q, k, v, g["sel"], g["todo"], B, 1.0, 1.0, 1.0,
                                    flips={(0, 65)})
    # key 65 rounds to 72 instead of 80 in the first step (then rescaled by
    # 1/1.5): l = 328 / 1.5 + 256 = 1424/3
    np.testing.assert_allclose(O1[0], [912 / 1424, 656 / 1424], atol=1e-12)
    assert abs(l1[0] - l0[0]) > 1e-3


def test_fp8_walk_order():
    """Steps of the walk: blocks backwards, a block's 64-key tiles descending,
    the short last block clipped, then the correction chunks; split u takes
    the CSR share [u c / U, (u + 1) c / U) and chunks u, u + U, ..."""
    steps = oracle.walk([0, 3, 5], [1, 2, 64, 130], 128, 700)
    got = [(kind, int(idx[0]), int(idx[-1])) if kind == "exact" else (kind, list(idx))
           for kind, idx in steps]
    assert got == [("exact", 640, 699), ("exact", 448, 511), ("exact", 384, 447),
                   ("exact", 64, 127), ("exact", 0, 63),
                   ("corr", [1, 2]), ("corr", [64]), ("corr", [130])]
    s0 = [(k, int(i[0])) if k == "exact" else (k, list(i)) for k, i in
          oracle.walk([0, 3, 5], [1, 2, 64, 130], 128, 700, 0, 2)]
    s1 = [(k, int(i[0])) if k == "exact" else (k, list(i)) for k, i in
          oracle.walk([0, 3, 5], [1, 2, 64, 130], 128, 700, 1, 2)]
    assert s0 == [("exact", 64), ("exact", 0), ("corr", [1, 2]), ("corr", [130])]
    assert s1 == [("exact", 640), ("exact", 448), ("exact", 384), ("corr", [64])]


@pytest.mark.parametrize("B,n_splits,correction", [(64, 1, True), (128, 1, True), (128, 3, True),
                                                   (64, 2, False), (128, 4, False)])
def test_fp8_walk_exact_arithmetic_equals_attend_rows(B, n_splits, correction):
    """With the rounding replaced by the identity, the walk, the running
    rescale, the 2^8 offset, the split combine and the LSE correction must
    reproduce plain block-sparse attention exactly."""
    rng = np.random.default_rng(21 + B + n_splits)
    L, d = 11 * B - 37, 8
    N = -(-L // B)
    # e4m3 codes times the per-tensor scales, as the fp8 inputs are
    k = oracle.e4m3_round(rng.standard_normal((L, d)) * 30) * 0.7 / 30
    v = oracle.e4m3_round(rng.standard_normal((L, d)) * 60) * 1.3 / 60
    kbar = oracle.pool_means(k[:, None], B)[:, 0]
    vbar = oracle.pool_means(v[:, None], B)[:, 0]
    I = N - 1
    pos = np.arange(I * B, L)
    q = rng.standard_normal((len(pos), d)) * 2
    sel = [0, 2, 3, 7, I]
    todo = oracle.todo_row(sel, I, correction)
    O, lse = oracle.attend_rows_fp8(pos, q, k, v, sel, todo, B, 0.4, 0.7 / 30, 1.3 / 60,
                                    n_splits=n_splits, quantize=lambda x: x)
    O2, lse2 = oracle.attend_rows(pos, q, k, v, kbar, vbar, sel, todo, B, 0.4)
    np.testing.assert_allclose(O, O2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_fp8_walk_probabilities_on_the_grid():
    """Every rounded probability is an e4m3 value in [0, 256], so numerator
    and l are sums of grid values; rounding only moves O within the e4m3
    spacing of the weights."""
    rng = np.random.default_rng(5)
    L, B, d = 256, 64, 4
    k = rng.standard_normal((L, d)) * 3
    v = rng.standard_normal((L, d))
    kbar = oracle.pool_means(k[:, None], B)[:, 0]
    vbar = oracle.pool_means(v[:, None], B)[:, 0]
    pos = np.arange(192, 256)
    q = rng.standard_normal((64, d)) * 3
    seen = []

    def spy(x):
        r = oracle.e4m3_round(x)
        seen.append(r)
        return r
    O, _ = oracle.attend_rows_fp8(pos, q, k, v, [1, 3], [0, 2], B, 1.0, 1.0, 1.0, quantize=spy)
    probs = np.concatenate([s.ravel() for s in seen[2:]])  # after kbar, vbar
    assert probs.max() <= 256 and probs.min() >= 0
    np.testing.assert_array_equal(oracle.e4m3_round(probs), probs)
    O2, _ = oracle.attend_rows(pos, q, k, v, kbar, vbar, [1, 3], [0, 2], B, 1.0)
    assert np.abs(O - O2).max() < 0.25  # rounding error of 3-bit weights, not a wrong term
