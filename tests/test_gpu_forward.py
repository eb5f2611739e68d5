"""dsa_forward (HIP) end to end: against the separate calls, against the CPU
oracle on the standard workloads (sampled rows where the oracle is slow)."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import (MIN_RECALL, TOL_ATTN_BF16, TOL_ATTN_F32, announce, host, oracle_attention_on, recall,
                       row_norm_err, rows_of)
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_03_amd import dsa as d
    return d


def _oracle_forward(p, rows=None, act=0):
    q_idx, w, q = rows_of(p, rows)
    return oracle.forward(p.cu_q_host, p.cu_k_host, q_idx, host(p.k_idx), w, q, host(p.kv), p.k, p.d_v, p.scale,
                          act=act, rows=rows)


def _check_rows(p, out, idx, rows, tol, need_exact_idx=False, act=0):
    rows = np.asarray(rows, np.int32)
    ri = torch.as_tensor(rows, dtype=torch.long, device=DEV)
    g_idx = idx[ri].cpu().numpy()
    g_out = out[ri].float().cpu().numpy()
    ref_out, ref_lse, _, ref_idx = _oracle_forward(p, rows, act=act)
    n = p.positions()[rows] + 1
    rec, rec_min = recall(g_idx, ref_idx, n)
    print(f"recall mean {rec:.5f} min {rec_min:.5f}")
    short = n <= p.k
    assert np.array_equal(g_idx[short], ref_idx[short])
    if need_exact_idx:
        assert np.array_equal(g_idx, ref_idx)
    assert rec >= MIN_RECALL
    # attention on the selection the GPU made
    o_on, _ = oracle_attention_on(p, g_idx, rows=rows)
    err = row_norm_err(g_out, o_on)
    print(f"attention row-normalised error {err:.3e}")
    assert err <= tol
    same = np.all(g_idx == ref_idx, axis=1)
    if same.any():
        assert row_norm_err(g_out[same], ref_out[same]) <= tol


def test_forward_equals_separate_calls(dsa):
    announce("forward vs separate calls")
    p = gen.make_problem("fwd", [3000, 2600], [3000, 1], H_I=64, H=64, k=512, device=DEV, seed=21)
    out, lse, idx = dsa.forward(p)
    scores = dsa.indexer_scores(p)
    idx2 = dsa.topk(p, scores)
    assert torch.equal(idx, idx2)
    out2, lse2 = dsa.sparse_mla_attn(p, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # chunking never changes the result
    out3, lse3, idx3 = dsa.forward(p, q_block=512)
    assert torch.equal(idx3, idx) and torch.equal(out3, out)


def test_forward_short_rows_masked_mode_with_key_splits(dsa):
    """Rows with pos + 1 <= k take the dense walk inside dsa_forward; with few
    rows the attention is split over keys, and the dense rows leave their later
    splits empty.  The outputs equal the separate calls bit for bit."""
    announce("forward masked mode with splits")
    p = gen.make_problem("fwd", [3000, 300, 500, 40], [1, 1, 2, 40], H_I=64, H=128, k=512, device=DEV, seed=27)
    out, lse, idx = dsa.forward(p)
    idx2 = dsa.topk(p, dsa.indexer_scores(p))
    assert torch.equal(idx, idx2)
    out2, lse2 = dsa.sparse_mla_attn(p, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_forward_integer_inputs_exact_selection(dsa):
    announce("forward integer inputs")
    p = gen.make_problem("fwd", [2500], [2500], H_I=64, H=128, k=256, integer=True, device=DEV, seed=22)
    out, _, idx = dsa.forward(p)
    rows = np.array([0, 255, 256, 257, 1000, 1777, 2499], np.int32)
    _check_rows(p, out, idx, rows, TOL_ATTN_BF16, need_exact_idx=True)


def test_forward_workgroups_mixing_skipped_and_live_rows(dsa):
    """k not a multiple of the indexer's 8-row workgroups and a row count that
    is not either: the workgroup holding rows 32..39 has rows that skip the
    indexer (pos + 1 <= k) next to rows that need it, and the last workgroup is
    partial; selections stay exact."""
    announce("forward mixed workgroups")
    p = gen.make_problem("fwd", [1003], [1003], H_I=64, H=32, k=37, integer=True, device=DEV, seed=26)
    out, _, idx = dsa.forward(p)
    idx2 = dsa.topk(p, dsa.indexer_scores(p))
    assert torch.equal(idx, idx2)
    rows = np.array([0, 31, 35, 36, 37, 38, 39, 40, 41, 500, 999, 1000, 1001, 1002], np.int32)
    _check_rows(p, out, idx, rows, TOL_ATTN_BF16, need_exact_idx=True)


@pytest.mark.parametrize("act", [0, 1])
def test_forward_random_inputs(dsa, act):
    announce("forward random", act)
    p = gen.make_problem("fwd", [4000, 1500], [4000, 2], H_I=64, H=128, k=1024, device=DEV, seed=23 + act)
    out, _, idx = dsa.forward(p, act=act)
    rows = np.array([0, 1023, 1024, 1025, 2222, 3999, 4000, 4001], np.int32)
    _check_rows(p, out, idx, rows, TOL_ATTN_BF16, act=act)


def test_tiny_fp32_config(dsa):
    announce("forward tiny_fp32")
    p = gen.make_config("tiny_fp32", device=DEV)
    out, _, idx = dsa.forward(p)
    _check_rows(p, out, idx, np.arange(p.total_q, dtype=np.int32), TOL_ATTN_F32)


def test_prefill_8k_config(dsa):
    announce("forward prefill_8k")
    p = gen.make_config("prefill_8k", device=DEV)
    out, _, idx = dsa.forward(p)
    _check_rows(p, out, idx, [0, 1, 2046, 2047, 2048, 2049, 4100, 6000, 8191], TOL_ATTN_BF16)


def test_decode_64x32k_config(dsa):
    announce("forward decode_64x32k")
    p = gen.make_config("decode_64x32k", device=DEV)
    out, _, idx = dsa.forward(p)
    _check_rows(p, out, idx, [0, 31, 63], TOL_ATTN_BF16)


def test_decode_mixed_config(dsa):
    announce("forward decode_mixed")
    p = gen.make_config("decode_mixed", device=DEV)
    out, _, idx = dsa.forward(p)
    _check_rows(p, out, idx, [0, 5, 31, 32, 39], TOL_ATTN_BF16)


def test_prefill_128k_config(dsa):
    announce("forward prefill_128k (bench launch configuration)")
    p = gen.make_config("prefill_128k", device=DEV)
    out, _, idx = dsa.forward(p)
    torch.cuda.synchronize()
    _check_rows(p, out, idx, [0, 2047, 2048, 65535, 131071], TOL_ATTN_BF16)
