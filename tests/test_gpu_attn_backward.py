"""Backward of the sparse MLA attention (HIP, dsa_sparse_mla_backward) against
the CPU oracle: dq and the latent rows' gradient (scatter-added)."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import announce, host, row_norm_err, rows_of
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"

# P and dS are rounded to bf16 for dkv's products (relative 2^-9), dS is a
# hi + lo bf16 pair for dq; the fp32 sums then carry about 2^-9 relative error
# at most: the bf16 attention bar
TOL_BWD = 1e-2


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_03_amd import dsa as d
    return d


def _subset_idx(seed, p, k):
    rng = np.random.default_rng(seed)
    pos = p.positions()
    idx = np.full((p.total_q, k), -1, np.int32)
    for i, ps in enumerate(pos):
        n = ps + 1
        sel = np.arange(n) if n <= k else np.sort(rng.choice(n, k, replace=False))
        idx[i, :len(sel)] = sel
    return idx


def _run(dsa, p, idx_h, seed):
    from sparse_attention_03_amd import libdsa as L
    idx = torch.from_numpy(idx_h).to(DEV)
    _, lse = dsa.sparse_mla_attn(p, idx)
    rng = np.random.default_rng(seed)
    dout_h = rng.standard_normal((p.total_q, p.H, p.d_v)).astype(np.float32)
    dout = torch.from_numpy(dout_h).to(DEV).to(torch.bfloat16)
    dq = torch.zeros((p.total_q, p.H, p.d_qk), dtype=torch.float32, device=DEV)
    dkv = torch.zeros((p.total_k, p.d_qk), dtype=torch.float32, device=DEV)
    b = L.batch_of(p)
    ws = torch.empty(max(L.dsa_sparse_mla_backward_workspace_size(b, p.H, idx_h.shape[1]), 16), dtype=torch.uint8,
                     device=DEV)
    L.dsa_sparse_mla_backward(b, p.q, p.kv, idx, p.d_v, p.scale, lse, dout, dq, dkv, ws)
    torch.cuda.synchronize()
    _, _, q = rows_of(p, None)
    rq, rk = oracle.sparse_mla_backward(p.cu_q_host, p.cu_k_host, q, host(p.kv), idx_h, p.d_v, p.scale,
                                        dout.float().cpu().numpy().astype(np.float64))
    return dq.cpu().numpy(), dkv.cpu().numpy(), rq, rk


@pytest.mark.parametrize("H,k", [(128, 256), (64, 2048), (32, 100)])
def test_attention_backward(dsa, H, k):
    announce("attention backward", H, k)
    p = gen.make_problem("ab", [3000, 150, 2500], [40, 1, 2], H_I=16, H=H, k=k, device=DEV, seed=100)
    idx_h = _subset_idx(101, p, k)
    dq, dkv, rq, rk = _run(dsa, p, idx_h, 102)
    e_q = row_norm_err(dq, rq)
    used = np.abs(rk).max(1) > 0
    e_k = row_norm_err(dkv[used], rk[used])
    print(f"row-normalised errors: dq {e_q:.2e} dkv {e_k:.2e} ({int(used.sum())} rows touched)")
    assert e_q <= TOL_BWD and e_k <= TOL_BWD
    assert np.all(dkv[~used] == 0.0)


def test_attention_backward_few_rows_split_over_keys(dsa):
    """Few rows: every row is split over its tiles (dq then adds with atomics)."""
    announce("attention backward, splits")
    p = gen.make_problem("ab", [20000, 9000], [1, 1], H_I=16, H=128, k=2048, device=DEV, seed=103)
    idx_h = _subset_idx(104, p, 2048)
    dq, dkv, rq, rk = _run(dsa, p, idx_h, 105)
    used = np.abs(rk).max(1) > 0
    assert row_norm_err(dq, rq) <= TOL_BWD
    assert row_norm_err(dkv[used], rk[used]) <= TOL_BWD
    assert np.all(dkv[~used] == 0.0)
