#!/usr/bin/env python3
"""Benchmark of the block-sparse prefill hot path on one MI355X.

One step = the whole path for one layer over one batch of synthetic inputs
already resident in HBM: pooling + block scores, selection, and block-sparse
attention with mean correction.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                    [--copy-calibration] [--evict-mib M] [--fp8-steps K8]

--copy-calibration ends the run with three plain device copies of 1 GiB, the
known-size reference that scales the FETCH_SIZE / WRITE_SIZE counters of a
rocprofv3 --pmc run of this same command into bytes.

Workload (default): 64K-token bf16 GQA prefill, Hq=32, Hkv=8, d=128, B=128,
alpha=0.05, sink 1 / window 2 / recent 1 blocks, mean correction on, inputs
from the seeded planted-block generator (block-clustered keys; every query
sums three visible block centres).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (CHUNK_BF16_64K, FP8_128K, GQA_BF16_16K, PAGED_VARLEN, SHARD_BF16_16K,  # noqa: E402
                       SWEEP_BF16_64K, TINY_F32, make_inputs)

METRIC = "sparse prefill ms/layer + dense-equiv TFLOP/s at 64K/128K (MFMA % of peak)"
CONFIGS = {
    "64k-bf16": SWEEP_BF16_64K,
    "128k-fp8": FP8_128K,
    "16k-bf16": GQA_BF16_16K,
    "paged-varlen": PAGED_VARLEN,
    "16k-tp8-shard": SHARD_BF16_16K,
    "64k-last-8k-chunk": CHUNK_BF16_64K,
    "tiny-f32": TINY_F32,
}
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# arithmetic type of the attention per input type: fp8 inputs multiply P V on
# the fp8 matrix cores (its attention fraction is taken against the fp8 peak)
COMPUTE_DTYPE = {"f32": "f32", "bf16": "bf16", "fp8": "fp8"}
ATTN_SOURCE = {dt: os.path.join(ROOT, "block_sparse_long_pooled_amd", "csrc", f)
               for dt, f in (("bf16", "attn_mfma.hip"), ("fp8", "attn_fp8.hip"),
                             ("f32", "attn_valu.hip"))}


def measured_traffic(workload: str, dtype: str):
    """HBM bytes per attention launch from the committed counter summary of
    this workload, or None when there is none or the attention kernel source
    has changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"attn_{dtype}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    with open(ATTN_SOURCE[dtype], "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def dense_flops(w) -> float:
    """QK^T + PV over the causal (query, key) pairs, every query head: query
    position p sees keys 0..p, the queries being the last Lq of L positions."""
    return 4.0 * w.d * w.hq * sum(L * (L + 1) / 2 - (L - Lq) * (L - Lq + 1) / 2
                                  for L, Lq in zip(w.seqlens, w.query_lens))


def effective_flops(w, cu: np.ndarray, idx: np.ndarray, correction: bool) -> tuple[float, float]:
    """Attention FLOPs the selection asks for: visible (query, key) pairs of
    the selected blocks (diagonal block counted causally) plus one pooled
    term per corrected block, times 4*d.  Returns (flops, density)."""
    pairs = 0.0
    sel_total = 0
    causal_total = 0
    seg = 0
    for L, Lq in zip(w.seqlens, w.query_lens):
        N = -(-L // w.block)
        qoff = L - Lq
        i0 = qoff // w.block if Lq else N
        n = N - i0  # tiles that hold a query
        for _h in range(w.hkv):
            I = np.arange(i0, N)
            c = cu[seg + 1:seg + n + 1] - cu[seg:seg + n]
            last = idx[np.maximum(cu[seg + 1:seg + n + 1] - 1, 0)]
            diag = (c > 0) & (last == I)
            q0 = np.maximum(I * w.block, qoff)
            nq = (np.minimum((I + 1) * w.block, L) - q0).astype(np.float64)
            before = (c - diag).astype(np.float64)  # selected full blocks J < I
            # row p of the diagonal block sees p - I*B + 1 of its keys
            dpairs = nq * (q0 - I * w.block) + nq * (nq + 1) / 2
            exact = nq * w.block * before + np.where(diag, dpairs, 0.0)
            todo = (I - before) if correction else np.zeros(n)
            pairs += float(np.sum(w.g * (exact + nq * todo)))
            sel_total += int(c.sum())
            causal_total += int(np.sum(I + 1))
            seg += n
    return 4.0 * w.d * pairs, sel_total / max(1, causal_total)


def cpu_baseline(w, inp, budget_s: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on the heaviest tiles of KV head 0,
    until the time budget is spent; reported as dense-equivalent TFLOP/s of
    the tiles it finished."""
    import oracle
    from oracle.fp8 import decode_e4m3fn

    def deq(t, scale):
        if w.dtype == "fp8":
            return decode_e4m3fn(t.numpy()) * scale
        return t.float().numpy().astype(np.float64)

    L = w.seqlens[0]
    qoff = L - w.query_lens[0]
    N = -(-L // w.block)
    h = 0
    kk = inp.k_logical if inp.k_logical is not None else inp.k
    vv = inp.v_logical if inp.v_logical is not None else inp.v
    k = deq(kk[:L, h:h + 1].contiguous(), inp.k_scale)
    v = deq(vv[:L, h:h + 1].contiguous(), inp.v_scale)
    t0 = time.time()
    kbar = oracle.pool_means(k, w.block)[:, 0]
    vbar = oracle.pool_means(v, w.block)[:, 0]
    t_pool = time.time() - t0
    done = []
    elapsed = t_pool
    for I in range(N - 1, qoff // w.block - 1, -1):
        q0 = max(I * w.block, qoff)
        nb = min((I + 1) * w.block, L) - q0
        # the tile's own rows, indexed from 0; positions shifted back afterwards
        q_tile = deq(inp.q[q0 - qoff:q0 - qoff + nb].contiguous(), inp.q_scale)
        t1 = time.time()
        pos, heads, rows = oracle.tile_query_rows(q_tile, h, w.g, w.block, 0)
        pos = pos + q0
        score = oracle.block_scores_row(rows, kbar, I, w.scale)
        sel, _ = oracle.select_row(score, I, w.alpha, w.sink, w.window, w.recent)
        todo = oracle.todo_row(sel, I, w.correction)
        oracle.attend_rows(pos, rows, k[:, 0], v[:, 0], kbar, vbar, sel, todo, w.block, w.scale)
        elapsed += time.time() - t1
        done.append((I, nb))
        if elapsed > budget_s and len(done) >= 2:
            break
    pairs = sum(w.g * (nb * (L - nb) + nb * (nb + 1) / 2) if I == N - 1 else
                w.g * (nb * ((I + 1) * w.block - nb) + nb * (nb + 1) / 2) for I, nb in done)
    flops = 4.0 * w.d * pairs
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(x.get("num_threads", 1)) for x in info)
    except Exception:  # noqa: BLE001
        pass
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"numpy float64 oracle (pool + scores + select + attention) on KV head 0, "
                   f"the {len(done)} heaviest query tiles I={done[-1][0]}..{done[0][0]} of "
                   f"{N}, {elapsed:.1f} s wall"),
    }


def stage_bytes_flops(w, sizes) -> dict:
    """Algorithmic work of each stage-1 kernel per launch (one layer).

    pool: K and V read once, K-bar and V-bar written (float32).
    scores: Q read once, K-bar read once, the score rows written; on the
    matrix cores every (row, pooled key) pair costs 2 d flops per bf16 term
    of the 2-term split of K-bar."""
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    pooled = int(sizes.pooled_rows)
    kv_bytes = 2 * w.total_tokens * w.hkv * w.d * esz
    pool = {"bytes": kv_bytes + 2 * pooled * w.hkv * w.d * 4}
    pairs = 0
    for L, Lq in zip(w.seqlens, w.query_lens):
        N = -(-L // w.block)
        i0 = (L - Lq) // w.block if Lq else N
        for I in range(i0, N):
            q0 = max(I * w.block, L - Lq)
            nq = min((I + 1) * w.block, L) - q0
            pairs += w.hkv * w.g * nq * (I + 1)
    scores = {"bytes": w.total_queries * w.hq * w.d * esz + pooled * w.hkv * w.d * 4 +
              int(sizes.score_elems) * 4,
              "mfma_flops": 2 * 2 * w.d * pairs if w.dtype != "f32" else 0}
    return {"pool": pool, "scores": scores}


def percentile(x, q):
    return float(np.percentile(np.asarray(x, dtype=np.float64), q))


def measure(bslp, torch, w, inp, steps: int, warmup: int, kv_splits: int, evict_bytes: int,
            v_dmajor: bool = False, evict_write: bool = False):
    """Runs the layer `warmup + steps` times with HIP events around each
    kernel launch on the launch stream; between steps a scratch buffer of
    evict_bytes is read (or, with evict_write, written) so the next step
    starts with cold caches (MALL and L2).  Reading evicts without leaving
    dirty lines, whose write-back would otherwise fall on the step's first
    kernel.  Returns per-step stage times (ms) and the buffers of the last
    step."""
    dev = torch.device("cuda")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    if v_dmajor:  # [Hkv, d, kv tokens] (contiguous K/V only here)
        v = v.permute(1, 2, 0).contiguous()
    table = torch.from_numpy(inp.table).to(dev) if inp.table is not None else None
    prob = bslp.make_problem(w.dtype, w.hq, w.hkv, w.d, w.block, w.query_lens,
                             softmax_scale=w.scale, q_scale=inp.q_scale, k_scale=inp.k_scale,
                             v_scale=inp.v_scale, page_table=table, page_size=w.page_size,
                             kv_splits=kv_splits,
                             kv_seqlens=w.seqlens if w.q_lens is not None else None,
                             v_dmajor=v_dmajor)
    params = bslp.make_params(w.alpha, w.sink, w.window, w.recent, w.correction)
    bufs = bslp.Buffers(prob)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    scratch = torch.zeros(max(4, evict_bytes) // 4, dtype=torch.float32, device=dev)

    def evict(i):
        if not evict_bytes:
            return
        if evict_write:
            scratch.fill_(float(i & 255))
        else:
            torch.sum(scratch)  # reads every byte once

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        bslp.pool_kv(prob, k, v, bufs.kbar, bufs.vbar, sp)
        rec(1)
        bslp.score_blocks(prob, q, bufs.kbar, bufs.scores, sp)
        rec(2)
        bslp.select_blocks(prob, params, q, bufs.kbar, bufs.scores, bufs.counts, bufs.cu, bufs.idx,
                           sp)
        rec(3)
        bslp.sparse_prefill_attn(prob, params, q, k, v, bufs.kbar, bufs.vbar, bufs.cu, bufs.idx,
                                 bufs.out, bufs.lse, bufs.workspace, sp)
        rec(4)

    for i in range(warmup):
        evict(i)
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evict(i + 1)  # outside the timed kernels
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])
    del scratch
    return dict(stage=stage, wall=wall, prob=prob, bufs=bufs, q=q, k=k, v=v, stream=stream, sp=sp,
                params=params)


def summarize(w, m, peak_attn: float) -> dict:
    """Median / p10 / p90 of the layer and of each kernel, the attention's
    effective flops and roofline fraction, and each stage-1 kernel's
    algorithmic bytes (and flops) against its roofs."""
    stage = m["stage"]
    layer = stage.sum(axis=1)
    med = np.median(stage, axis=0)
    bufs = m["bufs"]
    cu = bufs.cu.cpu().numpy().astype(np.int64)
    idx = bufs.idx.cpu().numpy().astype(np.int64)
    f_eff, density = effective_flops(w, cu, idx, w.correction)
    attn_ms = float(med[3])
    work = stage_bytes_flops(w, bufs.sizes)
    pool_ms, scores_ms = float(med[0]), float(med[1])
    pool_gbs = work["pool"]["bytes"] / (pool_ms * 1e-3) / 1e9
    sc = work["scores"]
    sc_gbs = sc["bytes"] / (scores_ms * 1e-3) / 1e9
    sc_tf = sc["mfma_flops"] / (scores_ms * 1e-3) / 1e12
    t_hbm = sc["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_mfma = sc["mfma_flops"] / (PEAK_TFLOPS["bf16"] * 1e12)
    achieved = f_eff / (attn_ms * 1e-3) / 1e12
    return {
        "layer_ms": {"median": float(np.median(layer)), "p10": percentile(layer, 10),
                     "p90": percentile(layer, 90), "mean": float(layer.mean())},
        "stages_ms": {"pool_kv": pool_ms, "block_scores": scores_ms, "select_blocks": float(med[2]),
                      "sparse_prefill_attn": attn_ms},
        "stages_p90_ms": {n: percentile(stage[:, j], 90) for j, n in
                          enumerate(("pool_kv", "block_scores", "select_blocks",
                                     "sparse_prefill_attn"))},
        "density": density,
        "attention": {"effective_flops": f_eff, "tflops": achieved, "peak": peak_attn,
                      "frac": achieved / peak_attn},
        "kernels": {
            "pool_kv": {"bound": "hbm", "bytes": work["pool"]["bytes"], "ms": pool_ms,
                        "gbs": pool_gbs, "frac": pool_gbs / PEAK_HBM_GBS},
            "block_scores": {"bound": "mfma" if t_mfma > t_hbm else "hbm",
                             "bytes": sc["bytes"], "mfma_flops_2term": sc["mfma_flops"],
                             "ms": scores_ms, "gbs": sc_gbs, "hbm_frac": sc_gbs / PEAK_HBM_GBS,
                             "mfma_tflops": sc_tf,
                             "mfma_frac": sc_tf / PEAK_TFLOPS["bf16"],
                             "roof_frac": max(t_hbm, t_mfma) / (scores_ms * 1e-3)},
        },
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="64k-bf16", choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kv-splits", type=int, default=0,
                    help="attention KV splits: 0 automatic, 1 none, 2..16 forced")
    ap.add_argument("--evict-mib", type=int, default=512,
                    help="scratch read between timed steps to evict MALL and L2 (0: none)")
    ap.add_argument("--evict-write", action="store_true",
                    help="write the eviction scratch instead of reading it (its dirty lines are "
                         "then written back during the next step's first kernel)")
    ap.add_argument("--quant-reps", type=int, default=5,
                    help="timed online e4m3 quantisations of Q for bf16 workloads (0 skips)")
    ap.add_argument("--dense-reps", type=int, default=3,
                    help="timed calls of the dense causal path (0 skips it)")
    ap.add_argument("--v-dmajor-ab", action="store_true",
                    help="also time the 128K fp8 workload with V given d-major")
    ap.add_argument("--fp8-steps", type=int, default=8,
                    help="timed steps of the 128K fp8 workload reported beside the default "
                         "64K bf16 one (0 skips it)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the layer has no "
              "cross-GPU step; across GPUs it shards by KV head or by request with no exchange.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_long_pooled_amd as bslp

    w = CONFIGS[args.config]
    t_gen = time.time()
    inp = make_inputs(w, args.seed)
    t_gen = time.time() - t_gen
    evict = args.evict_mib << 20
    cdt = COMPUTE_DTYPE[w.dtype]
    m = measure(bslp, torch, w, inp, args.steps, args.warmup, args.kv_splits, evict,
                evict_write=args.evict_write)
    sm = summarize(w, m, PEAK_TFLOPS[cdt])
    ms_step = sm["layer_ms"]["median"]
    f_dense = dense_flops(w)
    prob, bufs, q, k, v, stream, sp = (m[x] for x in ("prob", "bufs", "q", "k", "v", "stream", "sp"))
    dev = q.device
    res = {
        "metric": METRIC,
        "value": f_dense / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cdt,
        "data": "synthetic (seeded planted-block generator)",
        "config": {
            "workload": w.name, "seqlens": list(w.seqlens), "query_lens": list(w.query_lens),
            "hq": w.hq, "hkv": w.hkv,
            "input_dtype": w.dtype, "head_dim": w.d, "block": w.block, "alpha": w.alpha, "sink_blocks": w.sink,
            "window_blocks": w.window, "recent_blocks": w.recent,
            "mean_correction": bool(w.correction), "page_size": w.page_size,
            "kv_splits": args.kv_splits,
            "density": round(sm["density"], 5),
        },
        "ms_per_layer": ms_step,
        "timing": {"protocol": f"HIP events around each kernel launch on the launch stream; "
                               f"{args.evict_mib} MiB scratch {'written' if args.evict_write else 'read'} between steps (cold MALL/L2); "
                               f"median over {args.steps} steps",
                   "layer_ms": sm["layer_ms"], "stages_p90_ms": sm["stages_p90_ms"],
                   "wall_s": m["wall"]},
        "stages_ms": sm["stages_ms"],
        "roofline": {
            "kernel": "sparse_prefill_attn",
            "bound": "mfma",
            "achieved": sm["attention"]["tflops"],
            "peak": sm["attention"]["peak"],
            "unit": "TFLOP/s",
            "frac": sm["attention"]["frac"],
            "traffic": measured_traffic(w.name, w.dtype),
            "effective_flops": sm["attention"]["effective_flops"],
        },
        "kernels": sm["kernels"],
        "input_gen_s": round(t_gen, 2),
    }
    if args.dense_reps > 0:
        # the in-framework dense baseline: same kernel, every causal block
        dout = torch.empty_like(bufs.out)
        dlse = torch.empty_like(bufs.lse)
        bslp.dense_prefill_attn(prob, q, k, v, dout, dlse, sp)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.dense_reps):
            bslp.dense_prefill_attn(prob, q, k, v, dout, dlse, sp)
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / args.dense_reps
        dense_tf = f_dense / (dense_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[cdt]
        res["dense_attention"] = {"ms": dense_ms, "tflops": dense_tf, "frac": dense_tf / peak,
                                  "sparse_layer_speedup": dense_ms / ms_step}
        del dout, dlse
    if args.quant_reps > 0 and q.dtype == torch.bfloat16:
        # online per-tensor e4m3 quantisation of the workload's Q: amax pass,
        # then codes; 5 bytes per element (two reads of 2, one write of 1)
        codes = torch.empty(q.numel(), dtype=torch.uint8, device=dev)
        scale = torch.empty(1, dtype=torch.float32, device=dev)
        qflat = q.reshape(-1)
        bslp.quantize_e4m3(qflat, codes, scale, sp)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.quant_reps):
            bslp.quantize_e4m3(qflat, codes, scale, sp)
        d1.record(stream)
        torch.cuda.synchronize()
        qms = d0.elapsed_time(d1) / args.quant_reps
        gbs = 5.0 * q.numel() / (qms * 1e-3) / 1e9
        res["online_fp8_quant_q"] = {"elements": q.numel(), "ms": qms, "gbs": gbs,
                                     "frac_of_8TBs": gbs / PEAK_HBM_GBS}
        del codes, scale
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 1 << 30
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp)
    if args.fp8_steps > 0 and args.config == "64k-bf16":
        # the 128K half of the metric: the fp8 workload on the fp8 matrix
        # cores, same protocol; its attention fraction is against the fp8 peak
        del m, prob, bufs, q, k, v
        torch.cuda.empty_cache()
        w8 = CONFIGS["128k-fp8"]
        inp8 = make_inputs(w8, args.seed)
        m8 = measure(bslp, torch, w8, inp8, args.fp8_steps, 2, args.kv_splits, evict,
                     evict_write=args.evict_write)
        s8 = summarize(w8, m8, PEAK_TFLOPS["fp8"])
        res["fp8_128k"] = {
            "workload": w8.name, "density": round(s8["density"], 5),
            "ms_per_layer": s8["layer_ms"]["median"], "layer_ms": s8["layer_ms"],
            "stages_ms": s8["stages_ms"],
            "dense_equiv_tflops": dense_flops(w8) / (s8["layer_ms"]["median"] * 1e-3) / 1e12,
            "attention": s8["attention"], "kernels": s8["kernels"],
            "note": "P V on the fp8 matrix cores (e4m3 probabilities), Q K^T on the bf16 "
                    "matrix cores on exactly widened codes; frac against the 5 PF fp8 peak",
        }
        if args.v_dmajor_ab:
            # the same workload with V given d-major ([Hkv, d, kv tokens])
            del m8
            torch.cuda.empty_cache()
            md = measure(bslp, torch, w8, inp8, args.fp8_steps, 2, args.kv_splits, evict,
                         v_dmajor=True, evict_write=args.evict_write)
            sd = summarize(w8, md, PEAK_TFLOPS["fp8"])
            res["fp8_128k"]["v_dmajor"] = {"ms_per_layer": sd["layer_ms"]["median"],
                                           "stages_ms": sd["stages_ms"],
                                           "attention": sd["attention"]}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
