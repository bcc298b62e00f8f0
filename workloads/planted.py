"""Seeded synthetic prefill inputs with planted block structure.

This module only draws random numbers and converts dtypes; it holds none of
the attention arithmetic, so both the fp64 oracle and the GPU path can take
their inputs from it.

The shapes stand in for the long-context retrieval inputs the FlashPrefill V2
pages measure on (needle / RULER style prompts): keys are clustered around a
per-block centre, which gives the low intra-block variance the block-mean
proxy relies on (FlashPrefill V2, Sec. 3.1), and every query is the sum of a
few block centres, which plants a block-sparse attention pattern.  Optional
"vertical" key positions with a 4x larger norm plant the column pattern the
uniform probe queries are meant to catch.

Recipe per request b and KV head h (one PCG64 stream per (seed, b, h), fixed
draw order):

1. centres   c_J = sigma_c * N(0, I_d) for every key block J;
2. keys      k_j = c_{j // B} + key_noise * N(0, I_d);
3. values    v_j = N(0, I_d);
4. vertical  the keys at `vertical` positions, drawn once per request from the
             stream (seed, b) without replacement, are multiplied by 4;
5. attractor sets: if `attractors` is set, tile I gets min(attractors, I+1)
             distinct blocks from {0..I}, shared by the g query heads of h;
6. queries   for each query head of the group and each position i in tile I,
             `picks` blocks are drawn without replacement from the attractor
             set (or from {0..I}); if fewer blocks exist than picks they are
             drawn with replacement; q_i = sum of their centres
             + q_noise * N(0, I_d).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

FP8_E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """Shape, selection parameters and generator arguments of one prefill call."""

    name: str
    seqlens: tuple
    hq: int
    hkv: int
    d: int
    block: int
    dtype: str  # "f32" | "bf16" | "fp8"
    alpha: float = 0.05
    sink: int = 1
    window: int = 2
    recent: int = 1
    correction: bool = True
    sigma_c: float = 1.0
    key_noise: float = 0.3
    q_noise: float = 0.5
    picks: int = 3
    attractors: int | None = None
    vertical: int = 0
    page_size: int = 0  # 0: contiguous K/V
    seeds: tuple = (0,)
    # queries per request when they are only the last positions of its keys
    # (a chunk of a chunked prefill); None: every position is a query
    q_lens: tuple | None = None

    @property
    def g(self) -> int:
        return self.hq // self.hkv

    @property
    def query_lens(self) -> tuple:
        return tuple(self.q_lens) if self.q_lens is not None else tuple(self.seqlens)

    @property
    def total_queries(self) -> int:
        return int(sum(self.query_lens))

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five synthetic configurations.  Names say what they are.
TINY_F32 = Workload("tiny-f32-L2048-d64", (2048,), 1, 1, 64, 64, "f32",
                    seeds=(0, 1, 2, 3, 4))
GQA_BF16_16K = Workload("gqa-bf16-L16384-hq32-hkv8", (16384,), 32, 8, 128, 128,
                        "bf16", attractors=4, vertical=8, seeds=(0, 1))
SWEEP_BF16_64K = Workload("gqa-bf16-L65536-hq32-hkv8", (65536,), 32, 8, 128, 128,
                          "bf16")
FP8_128K = Workload("gqa-fp8-L131072-hq32-hkv4", (131072,), 32, 4, 128, 128, "fp8",
                    sigma_c=1.5)
PAGED_VARLEN = Workload("paged-varlen-6req-bf16-hq32-hkv8",
                        (4096, 8192, 32768, 65536, 131072, 262144), 32, 8, 128, 128,
                        "bf16", attractors=4, vertical=8, page_size=128)
# One GPU's share of the 16K GQA layer under 8-way head sharding: few work
# units, the case KV splitting is for.
SHARD_BF16_16K = Workload("tp8-shard-bf16-L16384-hq4-hkv1", (16384,), 4, 1, 128, 128, "bf16",
                          attractors=4, vertical=8)
# The last 8K-token chunk of a chunked 64K prefill: 8K queries over 64K keys.
CHUNK_BF16_64K = Workload("chunk8k-of-64k-bf16-hq32-hkv8", (65536,), 32, 8, 128, 128, "bf16",
                          q_lens=(8192,))
SWEEP_ALPHAS = (0.2, 0.1, 0.05, 0.025, 0.0125)


def _distinct_picks(rng: np.random.Generator, n: np.ndarray, k: int) -> np.ndarray:
    """For every entry of `n` draw k indices uniformly from range(n) without
    replacement (with replacement where n < k).  Vectorised sequential
    sampling: the t-th draw is uniform over the n - t unused values."""
    n = np.asarray(n, dtype=np.int64)
    u = rng.random((n.shape[0], k))
    out = np.empty((n.shape[0], k), dtype=np.int64)
    distinct = n >= k
    for t in range(k):
        avail = np.where(distinct, n - t, n)
        x = np.minimum((u[:, t] * avail).astype(np.int64), avail - 1)
        if t:
            # shift past the already-used values (ascending) so x lands on the
            # x-th unused value
            used = np.sort(out[:, :t], axis=1)
            for s in range(t):
                x = np.where(distinct & (x >= used[:, s]), x + 1, x)
        out[:, t] = x
    return out


def plant_head(seed: int, b: int, h: int, L: int, w: Workload, vpos: np.ndarray):
    """Draw q [L, g, d], k [L, d], v [L, d] (float32) for request b, KV head h."""
    B, d, g = w.block, w.d, w.g
    N = (L + B - 1) // B
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, h])))
    centres = (w.sigma_c * rng.standard_normal((N, d))).astype(np.float32)
    blk = np.arange(L) // B
    k = centres[blk] + np.float32(w.key_noise) * rng.standard_normal((L, d), dtype=np.float32)
    v = rng.standard_normal((L, d), dtype=np.float32)
    if vpos.size:
        k[vpos] *= np.float32(4.0)
    if w.attractors:
        avail = np.minimum(np.arange(N) + 1, w.attractors)
        att = _distinct_picks(rng, np.arange(N) + 1, w.attractors)  # [N, attractors]
    q = np.empty((L, g, d), dtype=np.float32)
    for hh in range(g):
        if w.attractors:
            sel = _distinct_picks(rng, avail[blk], w.picks)  # index into att row
            chosen = att[blk[:, None], sel]
        else:
            chosen = _distinct_picks(rng, blk + 1, w.picks)
        q[:, hh, :] = centres[chosen].sum(axis=1)
        q[:, hh, :] += np.float32(w.q_noise) * rng.standard_normal((L, d), dtype=np.float32)
    return q, k, v


def vertical_positions(seed: int, b: int, L: int, count: int) -> np.ndarray:
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))
    return np.sort(rng.choice(L, size=min(count, L), replace=False))


def generate_f32(w: Workload, seed: int, threads: int = 8):
    """Packed varlen float32 tensors: q [T, Hq, d], k [T, Hkv, d], v [T, Hkv, d]."""
    T = w.total_tokens
    q = np.empty((T, w.hq, w.d), dtype=np.float32)
    k = np.empty((T, w.hkv, w.d), dtype=np.float32)
    v = np.empty((T, w.hkv, w.d), dtype=np.float32)
    starts = np.concatenate([[0], np.cumsum(w.seqlens)]).astype(np.int64)

    jobs = []
    for b, L in enumerate(w.seqlens):
        vp = vertical_positions(seed, b, L, w.vertical)
        for h in range(w.hkv):
            jobs.append((b, h, L, vp))

    def run(job):
        b, h, L, vp = job
        qh, kh, vh = plant_head(seed, b, h, L, w, vp)
        s = starts[b]
        q[s:s + L, h * w.g:(h + 1) * w.g, :] = qh
        k[s:s + L, h, :] = kh
        v[s:s + L, h, :] = vh

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(run, jobs))
    return q, k, v


def page_table(w: Workload, seed: int):
    """Seeded random permutation of physical pages assigned to (request,
    logical page) in order.  Returns (table [num_seqs, max_pages] int32,
    num_physical_pages)."""
    p = w.page_size
    pages = [(L + p - 1) // p for L in w.seqlens]
    total = int(sum(pages))
    perm = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7919]))).permutation(total)
    table = np.zeros((len(pages), max(pages)), dtype=np.int32)
    o = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[o:o + n]
        o += n
    return table, total


@dataclass
class Inputs:
    """Device-ready tensors (torch, CPU) plus what the oracle needs."""

    w: Workload
    seed: int
    q: object  # torch tensor in the compute dtype (uint8 codes for fp8)
    k: object  # contiguous [T, Hkv, d] or paged [P*p, Hkv, d]
    v: object
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    table: np.ndarray | None = None
    k_logical: object = None  # contiguous copies when paged
    v_logical: object = None
    extra: dict = field(default_factory=dict)


def quantize_fp8(x_f32):
    """Per-tensor absmax scale; e4m3fn codes (torch uint8 view) and the scale."""
    import torch

    t = torch.from_numpy(x_f32) if isinstance(x_f32, np.ndarray) else x_f32
    amax = float(t.abs().max())
    scale = amax / FP8_E4M3_MAX if amax > 0 else 1.0
    codes = (t / scale).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), float(scale)


def make_inputs(w: Workload, seed: int, threads: int = 8) -> Inputs:
    import torch

    q, k, v = generate_f32(w, seed, threads)
    if w.q_lens is not None:  # keep the queries of the last positions
        starts = np.concatenate([[0], np.cumsum(w.seqlens)]).astype(np.int64)
        q = np.concatenate([q[starts[b] + L - Lq:starts[b] + L]
                            for b, (L, Lq) in enumerate(zip(w.seqlens, w.q_lens))])
    qs = ks = vs = 1.0
    if w.dtype == "f32":
        tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    elif w.dtype == "bf16":
        tq, tk, tv = (torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v))
    elif w.dtype == "fp8":
        tq, qs = quantize_fp8(q)
        tk, ks = quantize_fp8(k)
        tv, vs = quantize_fp8(v)
    else:
        raise ValueError(w.dtype)
    del q, k, v
    inp = Inputs(w, seed, tq, tk, tv, qs, ks, vs)
    if w.page_size:
        table, npages = page_table(w, seed)
        p = w.page_size
        shape = (npages * p, w.hkv, w.d)
        pk = torch.zeros(shape, dtype=tk.dtype)
        pv = torch.zeros(shape, dtype=tv.dtype)
        s = 0
        for b, L in enumerate(w.seqlens):
            for lp in range((L + p - 1) // p):
                n = min(p, L - lp * p)
                ph = int(table[b, lp])
                pk[ph * p:ph * p + n] = tk[s + lp * p:s + lp * p + n]
                pv[ph * p:ph * p + n] = tv[s + lp * p:s + lp * p + n]
            s += L
        inp.k_logical, inp.v_logical = tk, tv
        inp.k, inp.v, inp.table = pk, pv, table
    return inp
