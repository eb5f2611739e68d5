#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

One step = one dsa_forward over the 131072-token prefill (lightning indexer in
FP8 + causal top-k 2048 + sparse MLA attention over 128 heads, processed in
4096-query chunks), inputs resident in HBM.  Prints one JSON line:

  value            tokens/s of the 128K prefill (whole job, one GPU)
  roofline         dominant kernel: algorithmic work per step / its time per
                   step, against the MI355X dense MFMA peak of its dtype
  cpu_baseline     the CPU oracle on a bounded sample of the same workload,
                   extrapolated with the per-row cost model
  decode           the 64 x 32K decode batch: microseconds per token (cold:
                   caches flushed before each step; warm beside it)
  decode_mixed     the mixed-length decode batch, the same way
  prefill_8k       tokens/s of the 8192-token prefill
  length_sweep     prefill of L = 8K .. 128K tokens: step and per-kernel
                   times, log-log slopes against L

Per-kernel times come from a second, instrumented pass that issues the same
per-chunk launches through the individual C entry points with HIP events
between them on the launch stream.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp8": 5.0e15, "bf16": 2.5e15}   # MI355X dense MFMA, FLOP/s
HBM_PEAK = 8.0e12                         # bytes/s
CSRC = os.path.join(ROOT, "sparse_attention_03_amd", "csrc")
KERNEL_SOURCE = {"attention": ("sparse_mla.hip", "mla_tile.h", "dsa_common.h"), "indexer": ("indexer.hip", "dsa_common.h"),
                 "topk": ("topk.hip", "dsa_common.h")}
KERNEL_SYMBOL = {"attention": "mla_bf16_kernel", "indexer": "indexer_fp8_kernel", "topk": "topk_kernel"}
COPY_BYTES = 1 << 30                      # the calibration copy moves this many bytes each way


def source_sha(step):
    h = hashlib.sha256()
    for name in KERNEL_SOURCE[step]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(step):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE counter runs
    (profiles/traffic_<step>.json), or None if the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{step}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != source_sha(step):
        return None
    return t["bytes_per_launch"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_work(p):
    """Per step: indexer MFMA flops over the causal pairs of rows with n > k,
    attention flops over (query, selected entry) pairs, top-k bytes."""
    pos = p.positions().astype(np.int64)
    n = pos + 1
    big = n > p.k
    idx_pairs = int(n[big].sum())
    attn_pairs = int(np.minimum(n, p.k).sum())
    return dict(
        indexer_flops=idx_pairs * 2 * p.H_I * p.d_I,
        attention_flops=attn_pairs * 2 * p.H * (p.d_qk + p.d_v),
        topk_bytes=int((4 * n[big]).sum() + 4 * p.k * len(n)),
        indexer_pairs=idx_pairs, attention_pairs=attn_pairs)


def chunk_problem(p, r0, r1, skip_short):
    """The rows [r0, r1) of a one-sequence prefill as their own batch (same
    kernels and grids as a dsa_forward chunk).  With skip_short, rows whose
    candidates are all selected are left out, as dsa_forward does."""
    import torch
    from sparse_attention_03_amd import inputs as gen
    if skip_short:
        r0 = max(r0, p.k)
    c = gen.DSAInputs(name="chunk", cu_q=torch.tensor([0, r1 - r0], dtype=torch.int32, device=p.q.device),
                      cu_k=torch.tensor([0, r1], dtype=torch.int32, device=p.q.device),
                      cu_q_host=np.array([0, r1 - r0], np.int32), cu_k_host=np.array([0, r1], np.int32),
                      q_idx=p.q_idx[r0:r1], k_idx=p.k_idx, w=p.w[r0:r1], q=p.q[r0:r1], kv=p.kv, k=p.k, d_v=p.d_v,
                      scale=p.scale)
    return c


def kernel_times(p, reps=1):
    """Milliseconds per step spent in each step's kernels (HIP events)."""
    import torch
    from sparse_attention_03_amd import dsa, libdsa as L
    qb = p.q_block or 4096
    ev = lambda: torch.cuda.Event(enable_timing=True)
    tot = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    ld = dsa.score_ld(p.max_ctx)
    scores = torch.empty((qb, ld), dtype=torch.float32, device=p.q.device)
    n_ws = L.dsa_indexer_workspace_size(L.batch_of(chunk_problem(p, 0, min(p.total_q, qb), skip_short=False)), p.q_idx)
    idx_ws = torch.empty(max(n_ws, 16), dtype=torch.uint8, device=p.q.device)
    for _ in range(reps):
        for r0 in range(0, p.total_q, qb):
            r1 = min(p.total_q, r0 + qb)
            c_idx = chunk_problem(p, r0, r1, skip_short=True) if r1 > p.k else None
            c_all = chunk_problem(p, r0, r1, skip_short=False)
            e = [ev() for _ in range(4)]
            e[0].record()
            if c_idx is not None:
                L.dsa_indexer_scores(L.batch_of(c_idx), c_idx.q_idx, c_idx.k_idx, c_idx.w, scores, ws=idx_ws)
            e[1].record()
            idx = torch.empty((r1 - r0, p.k), dtype=torch.int32, device=p.q.device)
            L.dsa_topk(L.batch_of(c_all), scores, p.k, idx)
            e[2].record()
            out, lse = dsa.sparse_mla_attn(c_all, idx)
            e[3].record()
            torch.cuda.synchronize()
            tot["indexer"] += e[0].elapsed_time(e[1])
            tot["topk"] += e[1].elapsed_time(e[2])
            tot["attention"] += e[2].elapsed_time(e[3])
    return {k: v / reps for k, v in tot.items()}


def cpu_baseline(p, work, n_rows=640, seed=0):
    """Time the oracle on `n_rows` sampled rows of the same prefill and
    extrapolate to the whole step with the per-row cost model
    (t+1)*H_I*d_I (rows with n > k) + min(t+1, k)*H*(d_qk + d_v) MACs."""
    import oracle
    import torch
    from sparse_attention_03_amd import inputs as gen
    rng = np.random.default_rng(seed)
    T = p.total_q
    rows = np.sort(rng.choice(np.arange(T), n_rows, replace=False)).astype(np.int32)
    ri = torch.as_tensor(rows, dtype=torch.long, device=p.q.device)
    h = gen.storage_numpy
    args = (h(p.q_idx[ri]), h(p.k_idx), h(p.w[ri]), h(p.q[ri]), h(p.kv))

    def cost(t):
        t = np.asarray(t, np.int64)
        n = t + 1
        return np.where(n > p.k, n * p.H_I * p.d_I, 0) + np.minimum(n, p.k) * p.H * (p.d_qk + p.d_v)

    t0 = time.perf_counter()
    oracle.forward(p.cu_q_host, p.cu_k_host, *args, p.k, p.d_v, p.scale, rows=rows)
    dt = time.perf_counter() - t0
    rate = float(cost(rows).sum()) / dt                      # MAC/s of the oracle
    full = float(cost(np.arange(T)).sum()) / rate             # seconds for the whole step
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": T / full, "unit": "tokens/s", "cores": min(threads, os.cpu_count() or threads),
            "kind": "oracle",
            "sample": f"{n_rows} random rows of the 131072-token prefill (seed {seed}), {dt:.1f} s on the host; "
                      f"extrapolated to all rows with the per-row MAC cost model ({full:.0f} s per step)"}


DECODE_WORKLOADS = {
    "decode_64x32k": "64 sequences x 32768 cached tokens, 1 query each, k=2048",
    "decode_mixed": "32 sequences of U{4096..131072} cached tokens (seed 0) + 8 of 1024 (n <= k), 1 query each, k=2048",
}


def decode_kernel_us(p, reps=5, flush=None):
    """Microseconds per decode step in each step's kernels, through the
    separate entry points (the attention's time includes its split merge),
    mean of `reps` steps; with `flush` (a 1 GiB device buffer) it is written
    and read before each step, so every step starts with cold L2s and MALL
    (holding clean lines)."""
    import torch
    from sparse_attention_03_amd import dsa, libdsa as L
    ev = lambda: torch.cuda.Event(enable_timing=True)
    b = L.batch_of(p)
    scores = torch.empty((p.total_q, dsa.score_ld(p.max_ctx)), dtype=torch.float32, device=p.q.device)
    ws = torch.empty(max(L.dsa_indexer_workspace_size(b, p.q_idx), 16), dtype=torch.uint8, device=p.q.device)
    idx = torch.empty((p.total_q, p.k), dtype=torch.int32, device=p.q.device)
    tws = torch.empty(max(L.dsa_topk_workspace_size(b, p.k), 16), dtype=torch.uint8, device=p.q.device)
    tot = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    for i in range(reps + 1):
        if flush is not None:
            flush.fill_(float(i))
            flush.sum()
        e = [ev() for _ in range(4)]
        e[0].record()
        L.dsa_indexer_scores(b, p.q_idx, p.k_idx, p.w, scores, ws=ws)
        e[1].record()
        L.dsa_topk(b, scores, p.k, idx, ws=tws)
        e[2].record()
        dsa.sparse_mla_attn(p, idx)
        e[3].record()
        torch.cuda.synchronize()
        if i == 0:
            continue  # first pass: allocations
        for j, name in enumerate(tot):
            tot[name] += e[j].elapsed_time(e[j + 1]) * 1e3 / reps
    return tot


def decode_us_per_token(name="decode_64x32k", steps=20, warmup=3):
    """One decode step = dsa_forward over the batch (one new query per
    sequence).  Cold: before each timed step a 1 GiB buffer is written and
    then read, which evicts the L2s and the 256-MB MALL and leaves them
    holding clean lines of that buffer, so the step reads its caches from HBM;
    the step alone is bracketed by HIP events on the launch stream (median).
    After a write alone the caches hold 256 MB of the buffer's dirty lines,
    and the step also pays for writing them back: reported as well
    (cold_after_write_*).  Warm: `steps` back-to-back steps between two
    events."""
    import torch
    from sparse_attention_03_amd import dsa, inputs as gen
    p = gen.make_config(name, device="cuda")
    f = dsa.Forward(p)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    cold, dirty = [], []
    for i in range(2 * steps):
        flush.fill_(float(i))
        if i % 2 == 0:
            flush.sum()
        e0, e1 = ev(), ev()
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        (cold if i % 2 == 0 else dirty).append(e0.elapsed_time(e1) * 1e3)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(steps):
        f()
    e1.record()
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) * 1e3 / steps
    cold_us = float(np.median(cold))
    dirty_us = float(np.median(dirty))
    del f
    # the same kernels through the separate entry points, cold and warm (attention includes the split merge)
    kc = decode_kernel_us(p, flush=flush)
    kw = decode_kernel_us(p)
    del flush
    torch.cuda.empty_cache()
    return {"workload": f"{name}: {DECODE_WORKLOADS[name]}", "tokens_per_step": p.total_q,
            "us_per_token": cold_us / p.total_q, "us_per_step": cold_us,
            "timing": "cold (L2 and MALL flushed by a 1 GiB write and read), median",
            "cold_after_write_us_per_token": dirty_us / p.total_q, "cold_after_write_us_per_step": dirty_us,
            "warm_us_per_token": warm / p.total_q, "warm_us_per_step": warm,
            "cold_kernel_us": kc, "warm_kernel_us": kw}


def prefill_tokens_s(p, steps=5, warmup=1):
    """dsa_forward over a whole prefill: tokens/s and ms per step (HIP events)."""
    import torch
    from sparse_attention_03_amd import dsa
    f = dsa.Forward(p, with_idx=False, with_lse=False)
    for _ in range(warmup):
        f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del f
    return ms


def length_sweep(lengths, main=None):
    """Prefill of one sequence of L tokens (the prefill_8k distributions,
    4096-row chunks) for each L: ms per step of the whole dsa_forward and of
    each step's kernels, and log-log slopes of time against L.  The pages say
    the indexer stays quadratic in L while the attention becomes linear (each
    query attends to k = 2048 entries); the slopes test that.  `main`: the
    already measured 131072-token figures (reused, not measured again)."""
    import torch
    from sparse_attention_03_amd import inputs as gen
    rows = []
    for L in lengths:
        if main is not None and L == main["seq_len"]:
            rows.append(main)
            continue
        p = gen.make_problem("sweep", [L], [L], device="cuda", seed=0, q_block=4096)
        ms = prefill_tokens_s(p)
        kt = kernel_times(p)
        row = {"seq_len": L, "step_ms": ms, "tokens_s": L / ms * 1e3,
               "indexer_ms": kt["indexer"], "topk_ms": kt["topk"], "attention_ms": kt["attention"]}
        log("sweep", json.dumps(row))
        rows.append(row)
        del p
        torch.cuda.empty_cache()
    lx = np.log([r["seq_len"] for r in rows])
    slopes = {k: float(np.polyfit(lx, np.log([r[k] for r in rows]), 1)[0])
              for k in ("step_ms", "indexer_ms", "topk_ms", "attention_ms")}
    # the last doubling alone (the asymptotic slope of the attention is reached late: rows with n <= k cost less)
    last = {k: float(np.log(rows[-1][k] / rows[-2][k]) / np.log(rows[-1]["seq_len"] / rows[-2]["seq_len"]))
            for k in ("step_ms", "indexer_ms", "topk_ms", "attention_ms")} if len(rows) > 1 else {}
    return {"rows": rows, "loglog_slope_fit": slopes, "loglog_slope_last_doubling": last}


def crossover(lengths, steps=3, warmup=1):
    """Masked mode against the sparse path on one prefill sequence of each
    length (the prefill_8k distributions): ms per step of dsa_forward (indexer
    + top-k + sparse attention, 4096-row chunks) and of dsa_dense_mla_attn
    (dense causal MQA over the same rows, no indexer, no selection)."""
    import torch
    from sparse_attention_03_amd import dsa, inputs as gen, libdsa as L

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    rows = []
    for n in lengths:
        p = gen.make_problem("crossover", [n], [n], device="cuda", seed=0, q_block=4096)
        f = dsa.Forward(p, with_idx=False, with_lse=False)
        b = L.batch_of(p)
        out = torch.empty((p.total_q, p.H, p.d_v), dtype=p.q.dtype, device="cuda")
        nws = L.dsa_dense_mla_attn_workspace_size(b, L._dtype_code(p.q), p.H, p.d_qk, p.d_v)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
        sparse_ms = timed(f)
        dense_ms = timed(lambda: L.dsa_dense_mla_attn(b, p.q, p.kv, p.d_v, p.scale, out, None, ws=ws))
        row = {"seq_len": n, "sparse_ms": sparse_ms, "dense_ms": dense_ms,
               "sparse_tokens_s": n / (sparse_ms / 1e3), "dense_tokens_s": n / (dense_ms / 1e3)}
        log(json.dumps(row))
        rows.append(row)
        del p, f, out, ws
        torch.cuda.empty_cache()
    return rows


def append_bench(steps=10, warmup=2):
    """dsa_cache_append on a 131072-token prefill (fp32 indexer keys -> E4M3
    codes + E8M0 scales, bf16 latent rows copied) and on a 64-token decode
    step into a 64 x 32K cache; and the indexer's cost for per-token key
    scales on the prefill_128k and decode_64x32k workloads."""
    import torch
    from sparse_attention_03_amd import dsa, inputs as gen, libdsa as L

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {}
    n, d_I, d_qk = 131072, 128, 576
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    k32 = torch.randn((n, d_I), generator=g, device="cuda") / 11.3
    kbf = k32.to(torch.bfloat16)
    kv_new = torch.randn((n, d_qk), generator=g, device="cuda", dtype=torch.bfloat16)
    kc = torch.empty((n, d_I), dtype=torch.uint8, device="cuda")
    ks = torch.empty((n,), dtype=torch.uint8, device="cuda")
    kv_cache = torch.empty_like(kv_new)
    cases = {
        "keys_f32_scaled+latent_bf16": (dict(k_new=k32, k_cache=kc, k_scale=ks, kv_new=kv_new, kv_cache=kv_cache),
                                        n * (d_I * 4 + d_I + 1 + 2 * d_qk * 2)),
        "keys_f32_scaled": (dict(k_new=k32, k_cache=kc, k_scale=ks), n * (d_I * 4 + d_I + 1)),
        "keys_f32": (dict(k_new=k32, k_cache=kc), n * (d_I * 4 + d_I)),
        "keys_bf16_scaled": (dict(k_new=kbf, k_cache=kc, k_scale=ks), n * (d_I * 2 + d_I + 1)),
        "latent_bf16": (dict(kv_new=kv_new, kv_cache=kv_cache), n * 2 * d_qk * 2),
    }
    for name, (kw, nbytes) in cases.items():
        ms = timed(lambda: dsa.cache_append(**kw))
        res[f"prefill_{n}_{name}"] = {"ms": ms, "bytes": nbytes, "GB_s": nbytes / ms / 1e6,
                                      "frac_hbm": nbytes / ms * 1e3 / HBM_PEAK}
        log(name, json.dumps(res[f"prefill_{n}_{name}"]))
    del k32, kbf, kv_new, kc, ks, kv_cache
    torch.cuda.empty_cache()
    # decode: one new token per sequence, written at the end of its context
    B, ctx = 64, 32768
    kc = torch.empty((B * ctx, d_I), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B * ctx,), dtype=torch.uint8, device="cuda")
    kv_cache = torch.empty((B * ctx, d_qk), dtype=torch.bfloat16, device="cuda")
    dst = (torch.arange(1, B + 1, device="cuda", dtype=torch.int32) * ctx - 1).contiguous()
    k_new = torch.randn((B, d_I), generator=g, device="cuda")
    kv_new = torch.randn((B, d_qk), generator=g, device="cuda", dtype=torch.bfloat16)
    ms = timed(lambda: dsa.cache_append(k_new=k_new, k_cache=kc, k_scale=ks, kv_new=kv_new, kv_cache=kv_cache,
                                        dst_rows=dst))
    res["decode_64x32k_append"] = {"us_per_step": ms * 1e3}
    log("decode append", json.dumps(res["decode_64x32k_append"]))
    del kc, ks, kv_cache
    torch.cuda.empty_cache()
    # the indexer with and without per-token key scales (same codes)
    for cfg in ("prefill_128k", "decode_64x32k"):
        p = gen.make_config(cfg, device="cuda")
        ld = dsa.score_ld(p.max_ctx)
        scores = torch.empty((p.total_q, ld), dtype=torch.float32, device="cuda")
        b = L.batch_of(p)
        nws = L.dsa_indexer_workspace_size(b, p.q_idx)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
        sc = torch.full((p.total_k,), 127, dtype=torch.uint8, device="cuda")
        t_plain = timed(lambda: L.dsa_indexer_scores(b, p.q_idx, p.k_idx, p.w, scores, ws=ws))
        t_sc = timed(lambda: L.dsa_indexer_scores(b, p.q_idx, p.k_idx, p.w, scores, ws=ws, k_idx_scale=sc))
        res[f"indexer_{cfg}"] = {"unscaled_ms": t_plain, "scaled_ms": t_sc}
        log(cfg, json.dumps(res[f"indexer_{cfg}"]))
        del p, scores, ws, sc
        torch.cuda.empty_cache()
    return res


def align_bench(steps=5, warmup=1):
    """The indexer-alignment training kernels on one sequence of L tokens (all
    rows as queries, the prefill distributions): the sparse stage (target over
    the k = 2048 selected entries, KL, indexer backward) for L = 8192 and for a
    4096-row chunk of the 131072-token prefill, and the dense warm-up stage
    (target over every candidate, KL, backward) for L = 8192."""
    import torch
    from sparse_attention_03_amd import dsa, inputs as gen, libdsa as L

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {}
    for name, cfg, rows_from in (("prefill_8k", "prefill_8k", 0), ("prefill_128k_chunk", "prefill_128k", 131072 - 4096)):
        p = gen.make_config(cfg, device="cuda")
        if rows_from:
            # the last 4096 query rows of the sequence (every row has 2048 selected entries)
            n = p.total_q
            keep = slice(rows_from, n)
            p.q_idx, p.w, p.q = p.q_idx[keep].contiguous(), p.w[keep].contiguous(), p.q[keep].contiguous()
            p.cu_q = torch.tensor([0, n - rows_from], dtype=torch.int32, device="cuda")
            p.cu_q_host = np.array([0, n - rows_from], dtype=np.int32)
        b = L.batch_of(p)
        f = dsa.Forward(p)
        out, lse, idx = f()
        scores = dsa.indexer_scores(p, fill=0.0)
        T, k, H_I = p.total_q, p.k, p.H_I
        tgt = torch.empty((T, k), dtype=torch.float32, device="cuda")
        loss = torch.empty((T,), dtype=torch.float32, device="cuda")
        dI = torch.empty((T, k), dtype=torch.float32, device="cuda")
        dq = torch.zeros(p.q_idx.shape, dtype=torch.float32, device="cuda")
        dw = torch.zeros(p.w.shape, dtype=torch.float32, device="cuda")
        dk = torch.zeros(p.k_idx.shape, dtype=torch.float32, device="cuda")
        t_tgt = timed(lambda: L.dsa_attn_target(b, p.q, p.kv, p.scale, lse, tgt, idx=idx))
        t_kl = timed(lambda: L.dsa_indexer_kl(b, scores, tgt, loss, dI, idx=idx))
        t_bw = timed(lambda: L.dsa_indexer_backward(b, p.q_idx, p.k_idx, p.w, dI, dq, dw, dk, idx=idx))
        pairs = T * k
        r = {"rows": T, "k": k,
             "target_ms": t_tgt, "target_TFLOPs": pairs * p.H * 576 * 2 / t_tgt / 1e9,
             "kl_ms": t_kl, "kl_GBs": pairs * (4 + 4 + 4 + 4) / t_kl / 1e6,
             "backward_ms": t_bw, "backward_TFLOPs": pairs * H_I * 128 * 2 * 4 / t_bw / 1e9}
        res[f"sparse_{name}"] = r
        log("sparse", name, json.dumps(r))
        if not rows_from:
            # dense warm-up: every candidate
            ld = dsa.score_ld(p.max_ctx)
            _, lse_d = dsa.dense_mla_attn(p)
            tgt_d = torch.empty((T, ld), dtype=torch.float32, device="cuda")
            dI_d = torch.empty((T, ld), dtype=torch.float32, device="cuda")
            t_tgt = timed(lambda: L.dsa_attn_target(b, p.q, p.kv, p.scale, lse_d, tgt_d))
            t_kl = timed(lambda: L.dsa_indexer_kl(b, scores, tgt_d, loss, dI_d))
            t_bw = timed(lambda: L.dsa_indexer_backward(b, p.q_idx, p.k_idx, p.w, dI_d, dq, dw, dk))
            pairs = int((p.positions() + 1).sum())
            r = {"rows": T, "pairs": pairs,
                 "target_ms": t_tgt, "target_TFLOPs": pairs * p.H * 576 * 2 / t_tgt / 1e9,
                 "kl_ms": t_kl, "kl_GBs": pairs * (4 + 4 + 4 + 4) / t_kl / 1e6,
                 "backward_ms": t_bw, "backward_TFLOPs": pairs * H_I * 128 * 2 * 4 / t_bw / 1e9}
            res[f"dense_{name}"] = r
            log("dense", name, json.dumps(r))
            del tgt_d, dI_d
        del p, f, out, lse, idx, scores, tgt, dI, dq, dw, dk
        torch.cuda.empty_cache()
    return res


def attn_backward_bench(steps=3, warmup=1):
    """dsa_sparse_mla_backward on one sequence, all rows as queries, k = 2048,
    H = 128 (the prefill distributions, selections from dsa_forward, a random
    upstream gradient): L = 8192, and the last 4096 rows of the 131072-token
    prefill."""
    import torch
    from sparse_attention_03_amd import dsa, inputs as gen, libdsa as L

    res = {}
    for name, cfg, rows_from in (("prefill_8k", "prefill_8k", 0), ("prefill_128k_chunk", "prefill_128k", 131072 - 4096)):
        p = gen.make_config(cfg, device="cuda")
        if rows_from:
            n = p.total_q
            keep = slice(rows_from, n)
            p.q_idx, p.w, p.q = p.q_idx[keep].contiguous(), p.w[keep].contiguous(), p.q[keep].contiguous()
            p.cu_q = torch.tensor([0, n - rows_from], dtype=torch.int32, device="cuda")
            p.cu_q_host = np.array([0, n - rows_from], dtype=np.int32)
        b = L.batch_of(p)
        _, lse, idx = dsa.Forward(p)()
        g = torch.Generator(device="cuda")
        g.manual_seed(1)
        dout = torch.randn((p.total_q, p.H, p.d_v), generator=g, device="cuda", dtype=torch.bfloat16)
        dq = torch.zeros((p.total_q, p.H, p.d_qk), dtype=torch.float32, device="cuda")
        dkv = torch.zeros((p.total_k, p.d_qk), dtype=torch.float32, device="cuda")
        ws = torch.empty(L.dsa_sparse_mla_backward_workspace_size(b, p.H, p.k), dtype=torch.uint8, device="cuda")
        call = lambda: L.dsa_sparse_mla_backward(b, p.q, p.kv, idx, p.d_v, p.scale, lse, dout, dq, dkv, ws)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        # algorithmic: scores 576, dP 512, dq 576, dkv 576 + 512 multiply-adds per (row, entry, head)
        flop = p.total_q * p.k * p.H * 2 * (576 + 512 + 576 + 576 + 512)
        r = {"rows": p.total_q, "k": p.k, "H": p.H, "ms": ms, "TFLOPs": flop / ms / 1e9,
             "frac_bf16": flop / ms / 1e9 / 2500.0}
        res[name] = r
        log("attention backward", name, json.dumps(r))
        del p, lse, idx, dout, dq, dkv, ws
        torch.cuda.empty_cache()
    return res


def _short(name):
    m = re.search(r"dsa::\(anonymous namespace\)::(\w+)", name)
    if m:
        return m.group(1)
    name = name[5:] if name.startswith("void ") else name
    name = name.replace("(anonymous namespace)::", "")
    return re.split(r"[<(]", name, maxsplit=1)[0][-40:]


def _is_copy(path):
    """A counter file from `--copy-calibration`: its name or its folder's starts with copy."""
    return any(os.path.basename(p).startswith(("copy", "prof_copy")) for p in (path, os.path.dirname(path)))


def summarize(dirs, command, traffic_json=True):
    """Print a text summary of rocprofv3 output in `dirs` (kernel stats and, if
    present, counter collections, where files or folders named copy* or
    prof_copy* come from `--copy-calibration`); for FETCH_SIZE / WRITE_SIZE runs
    also write
    profiles/traffic_<step>.json for the kernels of the path (unless
    traffic_json is false: decode runs share kernel names with the prefill)."""
    out = []
    if command:
        out.append(f"command: {command}")
    files = lambda pat: sorted(f for d in dirs for f in glob.glob(os.path.join(d, "**", pat), recursive=True))
    for f in files("*kernel_stats.csv"):
        out.append(f"kernel stats ({os.path.basename(f)}):")
        out.append(f"  {'kernel':28s} {'calls':>6s} {'total ms':>10s} {'avg ms':>9s} {'min ms':>9s} {'max ms':>9s}")
        for r in csv.DictReader(open(f)):
            out.append(f"  {_short(r['Name']):28s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e6:10.3f} "
                       f"{float(r['AverageNs']) / 1e6:9.4f} {float(r['MinNs']) / 1e6:9.4f} {float(r['MaxNs']) / 1e6:9.4f}")
    for f in files("*kernel_trace.csv"):
        # the library's kernels per template instance and grid (one row per launch shape)
        shapes = {}
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            if "dsa::" not in name:
                continue
            m = re.search(r"(\w+)(<[^()]*>)?\(", name.replace("(anonymous namespace)::", ""))
            key = ((m.group(1) + (m.group(2) or "")) if m else name[:60], int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
                   int(r["Grid_Size_Y"]))
            shapes.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        if shapes:
            out.append(f"launch shapes ({os.path.basename(f)}):")
            out.append(f"  {'kernel':44s} {'grid':>14s} {'calls':>6s} {'avg us':>10s} {'min us':>10s}")
            for (k, gx, gy), v in shapes.items():
                out.append(f"  {k:44s} {f'{gx}x{gy}':>14s} {len(v):6d} {sum(v) / len(v):10.2f} {min(v):10.2f}")
    counters = {}
    other = {}     # (kernel instance, counter) -> [(value, ns)] for counters other than FETCH/WRITE
    for f in files("*counter_collection.csv"):
        if _is_copy(f):
            continue
        for r in csv.DictReader(open(f)):
            c = r["Counter_Name"]
            if c in ("FETCH_SIZE", "WRITE_SIZE") or "dsa::" not in r["Kernel_Name"]:
                continue
            m = re.search(r"(\w+)(<[^()]*>)?\(", r["Kernel_Name"].replace("(anonymous namespace)::", ""))
            key = m.group(1) + (m.group(2) or "") if m else _short(r["Kernel_Name"])
            other.setdefault((key, c), []).append(
                (float(r["Counter_Value"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    if other:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs: the clock is GUI_ACTIVE / 8 / kernel time, and the
        # MFMA pipes' busy share is SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GUI_ACTIVE / 8)
        names = sorted({c for _, c in other})
        out.append("counters per dispatch (mean), with the clock and the MFMA busy share where both are present:")
        out.append(f"  {'kernel':40s} {'n':>4s} " + " ".join(f"{c[:24]:>24s}" for c in names)
                   + f" {'GHz':>6s} {'MFMA busy':>9s}")
        for k in sorted({k for k, _ in other}):
            vals = {c: other.get((k, c), []) for c in names}
            mean = {c: (sum(v for v, _ in x) / len(x) if x else float("nan")) for c, x in vals.items()}
            n = max(len(x) for x in vals.values())
            ghz = busy = float("nan")
            gui = vals.get("GRBM_GUI_ACTIVE")
            if gui:
                ns = sum(t for _, t in gui) / len(gui)
                ghz = mean["GRBM_GUI_ACTIVE"] / 8 / ns if ns > 0 else float("nan")
                if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and mean["GRBM_GUI_ACTIVE"] > 0:
                    busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * mean["GRBM_GUI_ACTIVE"] / 8)
            out.append(f"  {k[:40]:40s} {n:4d} " + " ".join(f"{mean[c]:24.4g}" for c in names)
                       + f" {ghz:6.2f} {busy:9.3f}")
    for f in files("*counter_collection.csv"):
        calib = _is_copy(f)
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            if calib and "MulFunctor" not in name:
                continue
            key = "copy" if calib else _short(name)
            counters.setdefault((key, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    if any(c in ("FETCH_SIZE", "WRITE_SIZE") for _, c in counters):
        fac = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = counters.get(("copy", c), [])
            big = [v for v in vals if v * 1024 > COPY_BYTES / 2]
            if big:
                fac[c] = COPY_BYTES / (sum(big) / len(big) * 1024)
        out.append("counters (KiB per dispatch, mean over dispatches; copy calibration factor applied for bytes):")
        for step, sym in KERNEL_SYMBOL.items():
            fetch = counters.get((sym, "FETCH_SIZE"))
            write = counters.get((sym, "WRITE_SIZE"))
            if not fetch or not write:
                continue
            fk, wk = sum(fetch) / len(fetch), sum(write) / len(write)
            ff, wf = fac.get("FETCH_SIZE", 1.0), fac.get("WRITE_SIZE", 1.0)
            per_launch = fk * 1024 * ff + wk * 1024 * wf
            out.append(f"  {sym:28s} FETCH {fk:12.1f} KiB  WRITE {wk:12.1f} KiB  -> {per_launch / 1e9:8.3f} GB per launch")
            if not traffic_json:
                continue
            with open(os.path.join(ROOT, "profiles", f"traffic_{step}.json"), "w") as f:
                json.dump({"kernel": sym, "source_sha": source_sha(step), "bytes_per_launch": per_launch,
                           "fetch_kib_per_launch": fk, "write_kib_per_launch": wk, "fetch_factor": ff,
                           "write_factor": wf, "dispatches": len(fetch), "command": command}, f, indent=1)
        out.append(f"  copy calibration factors: {json.dumps(fac)} (bytes moved / counter bytes, 1 GiB copy)")
        # the same per template instance and launch size (workgroups), calibrated
        per = {}
        for f in files("*counter_collection.csv"):
            if _is_copy(f):
                continue
            for r in csv.DictReader(open(f)):
                c = r["Counter_Name"]
                if c not in ("FETCH_SIZE", "WRITE_SIZE") or "dsa::" not in r["Kernel_Name"]:
                    continue
                m = re.search(r"(\w+)(<[^()]*>)?\(", r["Kernel_Name"].replace("(anonymous namespace)::", ""))
                key = (m.group(1) + (m.group(2) or "") if m else _short(r["Kernel_Name"]),
                       int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
                per.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
        if per:
            out.append("  per instance and launch size (MB per dispatch, calibrated):")
            out.append(f"    {'kernel':44s} {'workgroups':>10s} {'n':>4s} {'read MB':>10s} {'write MB':>10s}")
            for (k, wg), d in sorted(per.items()):
                rd = sum(d.get("FETCH_SIZE", [0])) / max(1, len(d.get("FETCH_SIZE", []))) * 1024 * fac.get("FETCH_SIZE", 1.0)
                wr = sum(d.get("WRITE_SIZE", [0])) / max(1, len(d.get("WRITE_SIZE", []))) * 1024 * fac.get("WRITE_SIZE", 1.0)
                n = max(len(v) for v in d.values())
                out.append(f"    {k[:44]:44s} {wg:10d} {n:4d} {rd / 1e6:10.2f} {wr / 1e6:10.2f}")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-kernel-times", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip prefill_8k and the prefill length sweep")
    ap.add_argument("--decode-only", action="store_true", help="time only the 64 x 32K decode batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy 3 times (counter calibration under rocprofv3)")
    ap.add_argument("--crossover", metavar="L", type=int, nargs="+",
                    help="masked mode (dense attention) against the sparse path on one prefill sequence of each "
                         "length L, and exit")
    ap.add_argument("--attn-backward", action="store_true",
                    help="time the sparse attention backward, then exit")
    ap.add_argument("--align", action="store_true",
                    help="time the indexer-alignment kernels (target, KL, indexer backward), then exit")
    ap.add_argument("--append", action="store_true",
                    help="time dsa_cache_append (prefill and decode) and the indexer with key scales, then exit")
    ap.add_argument("--summarize", metavar="DIR", nargs="+", help="summarise rocprofv3 CSV output in DIR... and exit")
    ap.add_argument("--summary-command", default="", help="the command that produced DIR (recorded)")
    ap.add_argument("--no-traffic-json", action="store_true",
                    help="with --summarize: do not write profiles/traffic_<step>.json (for decode runs)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.summary_command, traffic_json=not args.no_traffic_json)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_03_amd import dsa, inputs as gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.crossover:
        print(json.dumps({"crossover": crossover(args.crossover, steps=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.attn_backward:
        print(json.dumps({"attn_backward": attn_backward_bench(steps=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.align:
        print(json.dumps({"align": align_bench(steps=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.append:
        print(json.dumps({"append": append_bench(steps=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.decode_only:
        print(json.dumps({name: decode_us_per_token(name, steps=args.steps, warmup=args.warmup)
                          for name in DECODE_WORKLOADS}), flush=True)
        return
    if args.copy_calibration:
        # an elementwise kernel (not hipMemcpy, which the counters do not see)
        # that reads COPY_BYTES and writes COPY_BYTES
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)
        return
    log("generating prefill_128k inputs on the GPU")
    p = gen.make_config("prefill_128k", device="cuda")
    f = dsa.Forward(p)
    work = algorithmic_work(p)
    log("warmup", args.warmup)
    for _ in range(args.warmup):
        f()
    torch.cuda.synchronize()
    log("timing", args.steps, "steps")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        f()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    log(f"{ms_step:.2f} ms/step (wall {wall / args.steps * 1e3:.2f} ms/step)")
    tokens_s = p.total_q / (ms_step / 1e3)

    result = {
        "metric": "DSA tokens/s (indexer+top-k+sparse MLA) at 128K prefill; decode us/token",
        "value": tokens_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / bf16 attention (fp32 accumulate)",
        "data": "synthetic, seeded (prefill_128k recipe)",
        "config": {"workload": "prefill_128k: 1 sequence, L=131072, H_I=64, d_I=128 fp8, k=2048, "
                               "H=128, d_qk=576, d_v=512 bf16, q_block=4096",
                   "seq_len": p.total_q, "q_block": p.q_block, "k": p.k},
    }
    if not args.no_kernel_times:
        log("instrumented pass (per-kernel HIP events)")
        kt = kernel_times(p)
        fl = {"indexer": (work["indexer_flops"], "fp8"), "attention": (work["attention_flops"], "bf16")}
        rows = {}
        for name, (flops, dt) in fl.items():
            ach = flops / (kt[name] / 1e3)
            rows[name] = {"ms_per_step": kt[name], "achieved_TFLOPs": ach / 1e12, "peak_TFLOPs": PEAK[dt] / 1e12,
                          "frac": ach / PEAK[dt]}
        tk_bw = work["topk_bytes"] / (kt["topk"] / 1e3)
        rows["topk"] = {"ms_per_step": kt["topk"], "achieved_GBs": tk_bw / 1e9, "peak_GBs": HBM_PEAK / 1e9,
                        "frac": tk_bw / HBM_PEAK}
        dom = max(("indexer", "attention"), key=lambda n: kt[n])
        d = rows[dom]
        launches = (p.total_q + (p.q_block or 4096) - 1) // (p.q_block or 4096)
        result["roofline"] = {"kernel": KERNEL_SYMBOL[dom], "bound": "mfma", "achieved": d["achieved_TFLOPs"],
                              "peak": d["peak_TFLOPs"], "unit": "TFLOP/s", "frac": d["frac"],
                              "traffic": stored_traffic(dom), "launches_per_step": launches,
                              "avg_launch_ms": kt[dom] / launches,
                              "flop_per_launch": fl[dom][0] / launches}
        result["kernels"] = rows
        log(json.dumps(rows))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on sampled rows)")
        result["cpu_baseline"] = cpu_baseline(p, work)
    main_row = None
    if "kernels" in result:
        main_row = {"seq_len": p.total_q, "step_ms": ms_step, "tokens_s": tokens_s,
                    "indexer_ms": result["kernels"]["indexer"]["ms_per_step"],
                    "topk_ms": result["kernels"]["topk"]["ms_per_step"],
                    "attention_ms": result["kernels"]["attention"]["ms_per_step"]}
    del f, p
    torch.cuda.empty_cache()
    if not args.no_decode:
        for name in DECODE_WORKLOADS:
            log(name)
            result["decode" if name == "decode_64x32k" else name] = decode_us_per_token(name)
    if not args.no_sweep:
        log("prefill_8k")
        p8 = gen.make_config("prefill_8k", device="cuda")
        ms8 = prefill_tokens_s(p8, steps=10, warmup=2)
        result["prefill_8k"] = {"workload": "prefill_8k: 1 sequence, L=8192, k=2048, H=128 (q_block 4096)",
                                "tokens_s": p8.total_q / ms8 * 1e3, "ms_per_step": ms8}
        del p8
        torch.cuda.empty_cache()
        if main_row is not None:
            log("length sweep")
            result["length_sweep"] = length_sweep([8192, 16384, 32768, 65536, 131072], main=main_row)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
