"""Shared helpers for the parity tests: copy a problem's bytes to the host for
the oracle, compare results, print what names each GPU case before it runs."""
import sys

import numpy as np
import torch

import oracle
from sparse_attention_03_amd import inputs as gen

# Tolerances of the acceptance bar.  The error is row-normalised: per row,
# max |gpu - ref| / max |ref|, and the worst row counts (score rows are per
# query, attention rows per (query, head)).  FP8 indexer scores: 2e-2 against
# the oracle on the same e4m3 bytes; bf16 attention: 1e-2; the fp32 tiny
# workload: 1e-5 for both; FP8 selection recall against the oracle's scores:
# 0.995 on rows with more than k candidates.
TOL_SCORES_FP8 = 2e-2
TOL_SCORES_F32 = 1e-5
TOL_ATTN_BF16 = 1e-2
TOL_ATTN_F32 = 1e-5
MIN_RECALL = 0.995


def announce(*what):
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def host(t):
    return gen.storage_numpy(t)


def rows_of(p, rows):
    """Query-side host arrays restricted to `rows` (all rows when None)."""
    if rows is None:
        return host(p.q_idx), host(p.w), host(p.q)
    ri = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=p.q_idx.device)
    return (host(p.q_idx.index_select(0, ri)), host(p.w.index_select(0, ri)), host(p.q.index_select(0, ri)))


def row_norm_err(got, ref, valid=None):
    """max over rows of max|got - ref| / max|ref| (rows = leading dims, last dim = row)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if valid is not None:
        got = np.where(valid, got, 0.0)
        ref = np.where(valid, ref, 0.0)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0


def causal_mask(p, rows, ld):
    pos = p.positions()[np.asarray(rows) if rows is not None else slice(None)]
    return np.arange(ld)[None, :] <= pos[:, None]


def recall(idx_gpu, idx_ref, n_valid):
    """Mean and minimum over rows with n > k of |S_gpu & S_ref| / k."""
    k = idx_gpu.shape[1]
    vals = []
    for a, b, n in zip(idx_gpu, idx_ref, n_valid):
        if n <= k:
            continue
        vals.append(len(np.intersect1d(a[a >= 0], b[b >= 0])) / k)
    if not vals:
        return 1.0, 1.0
    return float(np.mean(vals)), float(np.min(vals))


def oracle_attention_on(p, idx_rows, rows=None):
    """Oracle attention for `rows` given selected positions idx_rows [len(rows), k]."""
    _, _, q = rows_of(p, rows)
    return oracle.sparse_mla(p.cu_q_host, p.cu_k_host, q, host(p.kv), idx_rows, p.d_v, p.scale, rows=rows)
