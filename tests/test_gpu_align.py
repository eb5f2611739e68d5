"""Indexer alignment loss (HIP) against the CPU oracle: the target
distribution (dsa_attn_target), KL(p || softmax(I)) and its gradient
(dsa_indexer_kl)."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import announce, host, row_norm_err, rows_of
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"

# target: the exponent z - lse carries fp32 rounding of the score sum and of
# the given lse (|z|, |lse| up to ~20: a few 1e-6 absolute), which is the
# probability's relative error; measured about 2e-6, the bar is 10x that
TOL_TARGET = 2e-5
TOL_TARGET_F32 = 1e-5
# KL: fp32 terms and tree sums over up to 8K entries.  dI = (sum p) q - p with
# q = exp(I - lse): the fp32 lse (|lse| up to ~25 here) is off by up to
# |lse| 2^-23 ~ 3e-6, a relative error of q; dI values are at most 1
TOL_KL_LOSS = 1e-5
TOL_KL_GRAD = 1e-5


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_03_amd import dsa as d
    return d


def _lse_dense(dsa, p):
    _, lse = dsa.dense_mla_attn(p)
    return lse


def _target(dsa, p, lse, idx=None, ld=None):
    from sparse_attention_03_amd import libdsa as L
    m = p.max_ctx if idx is None else idx.shape[1]
    ld = (m + 31) // 32 * 32 if ld is None else ld
    out = torch.full((p.total_q, ld), float("nan"), dtype=torch.float32, device=DEV)
    L.dsa_attn_target(L.batch_of(p), p.q, p.kv, p.scale, lse, out, idx=idx)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("H", [24, 32, 64, 128])
def test_dense_target(dsa, H):
    announce("target dense", H)
    p = gen.make_problem("t", [700, 300, 1200, 65], [700, 3, 1, 65], H_I=16, H=H, k=64, device=DEV, seed=80)
    lse = _lse_dense(dsa, p)
    got = _target(dsa, p, lse)
    _, _, q = rows_of(p, None)
    ref = oracle.attn_target(p.cu_q_host, p.cu_k_host, q, host(p.kv), p.scale, ld=got.shape[1])
    pos = p.positions()
    valid = np.arange(got.shape[1])[None, :] <= pos[:, None]
    err = row_norm_err(got, ref, valid)
    print("row-normalised error", err)
    assert err <= TOL_TARGET
    tail = (np.arange(got.shape[1])[None, :] > pos[:, None]) & \
        (np.arange(got.shape[1])[None, :] < ((pos[:, None] + 1 + 31) // 32 * 32))
    assert np.all(got[tail] == 0.0)          # the rest of the last tile: written as 0
    np.testing.assert_allclose(np.where(valid, got, 0).sum(1), 1.0, atol=1e-4)


def _subset_idx(seed, p, k):
    rng = np.random.default_rng(seed)
    pos = p.positions()
    idx = np.full((p.total_q, k), -1, np.int32)
    for i, ps in enumerate(pos):
        n = ps + 1
        sel = np.arange(n) if n <= k else np.sort(rng.choice(n, k, replace=False))
        idx[i, :len(sel)] = sel
    return idx


@pytest.mark.parametrize("H,k", [(128, 256), (64, 2048), (32, 100)])
def test_selected_set_target(dsa, H, k):
    announce("target selected", H, k)
    p = gen.make_problem("t", [3000, 150, 2500], [40, 1, 2], H_I=16, H=H, k=k, device=DEV, seed=81)
    idx_h = _subset_idx(82, p, k)
    idx = torch.from_numpy(idx_h).to(DEV)
    _, lse = dsa.sparse_mla_attn(p, idx)
    got = _target(dsa, p, lse, idx=idx)
    _, _, q = rows_of(p, None)
    ref = oracle.attn_target(p.cu_q_host, p.cu_k_host, q, host(p.kv), p.scale, idx=idx_h)
    valid = idx_h >= 0
    err = row_norm_err(got[:, :k], ref, valid)
    print("row-normalised error", err)
    assert err <= TOL_TARGET
    assert np.all(got[:, :k][~valid] == 0.0)
    np.testing.assert_allclose(got[:, :k].sum(1), 1.0, atol=1e-4)


def test_selected_set_target_with_key_splits(dsa):
    """Few rows: the walk is split over keys (every split writes its own tiles)."""
    announce("target selected, splits")
    p = gen.make_problem("t", [20000, 9000], [1, 1], H_I=16, H=128, k=2048, device=DEV, seed=83)
    idx_h = _subset_idx(84, p, 2048)
    idx = torch.from_numpy(idx_h).to(DEV)
    _, lse = dsa.sparse_mla_attn(p, idx)
    got = _target(dsa, p, lse, idx=idx)
    _, _, q = rows_of(p, None)
    ref = oracle.attn_target(p.cu_q_host, p.cu_k_host, q, host(p.kv), p.scale, idx=idx_h)
    assert row_norm_err(got, ref, idx_h >= 0) <= TOL_TARGET


def test_tiny_fp32_target(dsa):
    announce("target fp32")
    p = gen.make_config("tiny_fp32", device=DEV)
    _, lse = dsa.dense_mla_attn(p)
    got = _target(dsa, p, lse)
    _, _, q = rows_of(p, None)
    ref = oracle.attn_target(p.cu_q_host, p.cu_k_host, q, host(p.kv), p.scale, ld=got.shape[1])
    valid = np.arange(got.shape[1])[None, :] <= p.positions()[:, None]
    assert row_norm_err(got, ref, valid) <= TOL_TARGET_F32
    idx_h = _subset_idx(85, p, 32)
    idx = torch.from_numpy(idx_h).to(DEV)
    _, lse = dsa.sparse_mla_attn(p, idx)
    got = _target(dsa, p, lse, idx=idx)
    ref = oracle.attn_target(p.cu_q_host, p.cu_k_host, q, host(p.kv), p.scale, idx=idx_h)
    assert row_norm_err(got[:, :32], ref, idx_h >= 0) <= TOL_TARGET_F32


def _kl_inputs(seed, p, m, idx_h=None):
    """Synthetic index scores (by position) and targets (by entry)."""
    rng = np.random.default_rng(seed)
    ld = (p.max_ctx + 63) // 64 * 64
    scores = (rng.standard_normal((p.total_q, ld)) * 4).astype(np.float32)
    tgt = (rng.random((p.total_q, m)) ** 4).astype(np.float32)
    tgt[:, 1::7] = 0.0
    pos = p.positions()
    for i, ps in enumerate(pos):
        valid = (np.arange(m) <= ps) if idx_h is None else (idx_h[i] >= 0)
        tgt[i, ~valid] = 0.0
        tgt[i] /= max(tgt[i].sum(), 1e-30)
    return scores, tgt


def _kl_call(p, scores, tgt, idx=None):
    from sparse_attention_03_amd import libdsa as L
    s_d = torch.from_numpy(scores).to(DEV)
    p_d = torch.from_numpy(tgt).to(DEV)
    loss = torch.full((p.total_q,), float("nan"), dtype=torch.float32, device=DEV)
    dI = torch.full(tgt.shape, float("nan"), dtype=torch.float32, device=DEV)
    L.dsa_indexer_kl(L.batch_of(p), s_d, p_d, loss, dI, idx=idx)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), dI.cpu().numpy()


def test_kl_dense(dsa):
    announce("kl dense")
    p = gen.make_problem("kl", [5000, 300, 8000], [5000, 2, 1], H_I=16, H=32, k=64, device=DEV, seed=86)
    m = (p.max_ctx + 63) // 64 * 64
    scores, tgt = _kl_inputs(87, p, m)
    loss, dI = _kl_call(p, scores, tgt)
    pos = p.positions()
    ref_loss, ref_dI = oracle.indexer_kl(scores[:, :m], tgt, pos + 1)
    rel = np.abs(loss - ref_loss) / np.maximum(np.abs(ref_loss), 1.0)
    print("loss rel error", rel.max())
    assert rel.max() <= TOL_KL_LOSS
    valid = np.arange(m)[None, :] <= pos[:, None]
    assert np.max(np.abs(np.where(valid, dI - ref_dI, 0.0))) <= TOL_KL_GRAD
    assert np.all(np.isnan(dI[~valid]))       # entries past the causal bound are not written


def test_kl_selected_set(dsa):
    announce("kl selected")
    p = gen.make_problem("kl", [3000, 100, 2600], [300, 1, 2], H_I=16, H=32, k=512, device=DEV, seed=88)
    k = 512
    idx_h = _subset_idx(89, p, k)
    scores, tgt = _kl_inputs(90, p, k, idx_h)
    loss, dI = _kl_call(p, scores, tgt, idx=torch.from_numpy(idx_h).to(DEV))
    gathered = np.take_along_axis(scores, np.maximum(idx_h, 0), axis=1)
    cnt = (idx_h >= 0).sum(1)
    ref_loss, ref_dI = oracle.indexer_kl(gathered, tgt, cnt)
    rel = np.abs(loss - ref_loss) / np.maximum(np.abs(ref_loss), 1.0)
    assert rel.max() <= TOL_KL_LOSS
    assert np.max(np.abs(dI - ref_dI)) <= TOL_KL_GRAD     # non-candidate entries: 0 on both sides


# ------------------------------------------------------- indexer backward

# dq and dk: g w act'(x) is rounded to bf16 (relative 2^-9) for the two
# products, whose fp32 sums then carry about that relative error against the
# terms' magnitudes; the bar is the bf16 attention bar.  dw is fp32 throughout.
TOL_BWD_BF16 = 1e-2
TOL_BWD_DW = 1e-5


def _bwd_call(p, g_np, act=0, idx=None):
    from sparse_attention_03_amd import libdsa as L
    g_d = torch.from_numpy(g_np).to(DEV)
    dq = torch.zeros(p.q_idx.shape, dtype=torch.float32, device=DEV)
    dw = torch.zeros(p.w.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(p.k_idx.shape, dtype=torch.float32, device=DEV)
    L.dsa_indexer_backward(L.batch_of(p), p.q_idx, p.k_idx, p.w, g_d, dq, dw, dk, act=act, idx=idx,
                           k_idx_scale=p.k_idx_scale)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dw.cpu().numpy(), dk.cpu().numpy()


def _bwd_oracle(p, g_np, act=0, idx_h=None):
    q_idx, w, _ = rows_of(p, None)
    return oracle.indexer_backward(p.cu_q_host, p.cu_k_host, q_idx, host(p.k_idx), w, g_np.astype(np.float64),
                                   act=act, idx=idx_h,
                                   k_scale=None if p.k_idx_scale is None else host(p.k_idx_scale))


def _upstream(seed, p, m, integer, idx_h=None):
    rng = np.random.default_rng(seed)
    g = rng.integers(-4, 5, (p.total_q, m)).astype(np.float32) if integer else \
        rng.standard_normal((p.total_q, m)).astype(np.float32)
    pos = p.positions()
    for i, ps in enumerate(pos):
        valid = (np.arange(m) <= ps) if idx_h is None else (idx_h[i] >= 0)
        g[i, ~valid] = 0.0
    return g


@pytest.mark.parametrize("H_I", [16, 20, 64])
@pytest.mark.parametrize("mode", ["dense", "selected"])
def test_indexer_backward_integer_exact(dsa, H_I, mode):
    """Integer inputs and upstream: g w act'(x) is exact in bf16 and every sum
    is exact in fp32 in any order, so all three gradients are bit-exact."""
    announce("indexer backward integer", H_I, mode)
    p = gen.make_problem("bw", [300, 77, 1000, 129], [300, 5, 3, 64], H_I=H_I, H=32, k=64, integer=True,
                         device=DEV, seed=91)
    idx_h = _subset_idx(92, p, 64) if mode == "selected" else None
    m = (p.max_ctx + 63) // 64 * 64 if idx_h is None else 64
    g = _upstream(93, p, m, True, idx_h)
    idx = None if idx_h is None else torch.from_numpy(idx_h).to(DEV)
    dq, dw, dk = _bwd_call(p, g, idx=idx)
    rq, rw, rk = _bwd_oracle(p, g, idx_h=idx_h)
    assert np.array_equal(dq, rq.astype(np.float32))
    assert np.array_equal(dw, rw.astype(np.float32))
    assert np.array_equal(dk, rk.astype(np.float32))


def _drop_ambiguous_relu(p, g, idx_h):
    """ReLU's slope steps at x = 0, so where x lies within the fp32 rounding of
    the kernel's sum (|x| <= 2^-17 sum |q_d k_d|: 128 products, fp32) the two
    sides may take different branches.  Such (row, key) pairs get g = 0, so
    every decision that counts is the same on both sides."""
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    q = vals[host(p.q_idx)]
    k = vals[host(p.k_idx)]
    pos, base = p.positions(), p.cu_k_host[:-1][np.searchsorted(p.cu_q_host, np.arange(p.total_q), "right") - 1]
    dropped = 0
    for i in range(p.total_q):
        sel = np.arange(pos[i] + 1) if idx_h is None else idx_h[i][idx_h[i] >= 0]
        ent = sel if idx_h is None else np.nonzero(idx_h[i] >= 0)[0]
        kk = k[base[i] + sel]
        x = q[i] @ kk.T
        band = 2.0 ** -17 * (np.abs(q[i]) @ np.abs(kk).T)
        amb = np.any(np.abs(x) <= band, axis=0)
        g[i, ent[amb]] = 0.0
        dropped += int(amb.sum())
    print("ambiguous (row, key) pairs dropped:", dropped)
    return g


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("mode", ["dense", "selected"])
def test_indexer_backward_random(dsa, act, mode):
    announce("indexer backward random", act, mode)
    p = gen.make_problem("bw", [2000, 300, 700], [400, 2, 1], H_I=64, H=32, k=256, device=DEV, seed=94)
    idx_h = _subset_idx(95, p, 256) if mode == "selected" else None
    m = (p.max_ctx + 63) // 64 * 64 if idx_h is None else 256
    g = _upstream(96, p, m, False, idx_h)
    if act == 0:
        g = _drop_ambiguous_relu(p, g, idx_h)
    idx = None if idx_h is None else torch.from_numpy(idx_h).to(DEV)
    dq, dw, dk = _bwd_call(p, g, act=act, idx=idx)
    rq, rw, rk = _bwd_oracle(p, g, act=act, idx_h=idx_h)
    e_q = row_norm_err(dq, rq)
    e_w = row_norm_err(dw, rw)
    used = np.abs(rk).max(1) > 0
    e_k = row_norm_err(dk[used], rk[used])
    print(f"row-normalised errors: dq {e_q:.2e} dw {e_w:.2e} dk {e_k:.2e}")
    assert e_q <= TOL_BWD_BF16 and e_k <= TOL_BWD_BF16 and e_w <= TOL_BWD_DW
    assert np.all(dk[~used] == 0.0)


def test_indexer_backward_scaled_keys(dsa):
    announce("indexer backward scaled keys")
    p = gen.make_problem("bw", [900, 40], [200, 1], H_I=32, H=32, k=128, integer=True, device=DEV, seed=97)
    rng = np.random.default_rng(98)
    p.k_idx_scale = torch.from_numpy(rng.integers(124, 131, p.total_k).astype(np.uint8)).to(DEV)
    m = (p.max_ctx + 63) // 64 * 64
    g = _upstream(99, p, m, True)
    dq, dw, dk = _bwd_call(p, g)
    rq, rw, rk = _bwd_oracle(p, g)
    assert np.array_equal(dq, rq.astype(np.float32))
    assert np.array_equal(dw, rw.astype(np.float32))
    assert np.array_equal(dk, rk.astype(np.float32))
