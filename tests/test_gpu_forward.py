"""dsa_forward (HIP) end to end: against the separate calls and against the CPU
oracle on ragged batches (the five standard workloads are in
test_gpu_configs.py)."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import (MIN_RECALL, TOL_ATTN_BF16, announce, host, oracle_attention_on, recall,
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
    assert rec >= MIN_RECALL and rec_min >= 0.99
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


@pytest.mark.parametrize("act", [0, 1])
def test_forward_short_last_chunk_scores_as_the_batch(dsa, act):
    """A prefill-like batch whose last chunk holds fewer than 8 rows per
    sequence: the indexer keeps the batch's form for that chunk, so on random
    inputs the selection equals the separate calls over the whole batch bit
    for bit.  (The attention of such a short chunk is split over keys, while
    the one call over the whole batch is not, so there the outputs agree to
    rounding, not bit for bit.)"""
    announce("forward short last chunk", act)
    p = gen.make_problem("fwd", [3001, 2600], [3001, 1], H_I=64, H=128, k=512, device=DEV, seed=28 + act)
    idx_ref = dsa.topk(p, dsa.indexer_scores(p, act=act))
    out_ref, lse_ref = dsa.sparse_mla_attn(p, idx_ref)
    for qb in (1000, 3000, 997):       # last chunks of 2, 2 and 10 rows
        out, lse, idx = dsa.forward(p, act=act, q_block=qb)
        assert torch.equal(idx, idx_ref), qb
        assert row_norm_err(out.float().cpu().numpy(), out_ref.float().cpu().numpy()) <= TOL_ATTN_BF16, qb
        assert float((lse - lse_ref).abs().max()) <= 1e-3, qb
        n_full = (p.total_q // qb) * qb  # rows of whole chunks: the same split as the one call
        assert torch.equal(out[:n_full], out_ref[:n_full]), qb


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


def test_forward_head_counts_not_multiples_of_32_or_16(dsa):
    """16 query heads and 12 indexer heads (a sharded model's share, say):
    exact selections on integer inputs and attention within the bf16 bar."""
    announce("forward H=16, H_I=12")
    p = gen.make_problem("fwd", [1500, 900], [1500, 2], H_I=12, H=16, k=256, integer=True, device=DEV, seed=29)
    out, _, idx = dsa.forward(p)
    idx2 = dsa.topk(p, dsa.indexer_scores(p))
    assert torch.equal(idx, idx2)
    rows = np.array([0, 255, 256, 900, 1499, 1500, 1501], np.int32)
    _check_rows(p, out, idx, rows, TOL_ATTN_BF16, need_exact_idx=True)


@pytest.mark.parametrize("act", [0, 1])
def test_forward_long_rows_random(dsa, act):
    """One long sequence (rows of up to 12000 candidates, 24 times k) in the
    default chunks and in chunks of 3000 rows: the selection equals the
    separate calls bit for bit."""
    announce("forward long rows, random", act)
    p = gen.make_problem("fwd", [12000], [12000], H_I=64, H=32, k=512, device=DEV, seed=40 + act)
    idx_ref = dsa.topk(p, dsa.indexer_scores(p, act=act))
    for qb in (0, 3000):
        _, _, idx = dsa.forward(p, act=act, q_block=qb)
        assert torch.equal(idx, idx_ref), qb


def test_forward_long_rows_ties(dsa):
    """Integer inputs: long rows whose scores hold many exact ties, so the
    k-th place is a tie that goes to the lower positions; the selection equals
    the separate calls and the oracle."""
    announce("forward long rows, ties")
    p = gen.make_problem("fwd", [9000, 7000], [9000, 300], H_I=64, H=32, k=384, integer=True, device=DEV, seed=42)
    out, _, idx = dsa.forward(p)
    idx_ref = dsa.topk(p, dsa.indexer_scores(p))
    assert torch.equal(idx, idx_ref)
    rows = np.array([3071, 3072, 3073, 5000, 8999, 9000, 9150, 9299], np.int32)
    _check_rows(p, out, idx, rows, TOL_ATTN_BF16, need_exact_idx=True)


def test_forward_nan_keys(dsa):
    """Keys holding the E4M3 NaN code give NaN scores, which rank below every
    number: rows select exactly what the separate calls select."""
    announce("forward NaN keys")
    p = gen.make_problem("fwd", [10000], [10000], H_I=64, H=32, k=512, device=DEV, seed=43)
    kb = p.k_idx.view(torch.uint8)
    kb[::37, 5] = 0x7F            # NaN in one element of every 37th key
    kb[4096:4104, :] = 0x7F       # eight NaN keys in a row
    idx_ref = dsa.topk(p, dsa.indexer_scores(p))
    _, _, idx = dsa.forward(p)
    assert torch.equal(idx, idx_ref)


def test_forward_narrow_indexer_keys(dsa):
    """d_I = 64 (FP8): the forward widens the keys once and each chunk's
    queries, and selects what the separate calls select; integer inputs,
    exact against the oracle."""
    announce("forward d_I = 64")
    p = gen.make_problem("fwd", [2500, 1200], [2500, 3], H_I=32, d_I=64, H=32, k=256, integer=True, device=DEV,
                         seed=44)
    for qb in (0, 700):
        out, _, idx = dsa.forward(p, q_block=qb)
        assert torch.equal(idx, dsa.topk(p, dsa.indexer_scores(p))), qb
    rows = np.array([0, 255, 256, 1999, 2499, 2500, 2502], np.int32)
    _check_rows(p, out, idx, rows, TOL_ATTN_BF16, need_exact_idx=True)


def test_forward_narrow_attention_widths(dsa):
    """d_qk = 192, d_v = 128 (BF16): the forward widens the latent once and
    each chunk's queries, stages the output and keeps its first d_v columns;
    equal to the separate calls, with and without key splits."""
    announce("forward attention widths")
    p = gen.make_problem("fwd", [3000, 2600], [3000, 1], H_I=64, H=64, d_qk=192, d_v=128, k=512, device=DEV,
                         seed=45)
    out, lse, idx = dsa.forward(p)
    idx2 = dsa.topk(p, dsa.indexer_scores(p))
    assert torch.equal(idx, idx2)
    out2, lse2 = dsa.sparse_mla_attn(p, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    out3, lse3, idx3 = dsa.forward(p, q_block=1000)
    assert torch.equal(idx3, idx)
    assert row_norm_err(out3.float().cpu().numpy(), out.float().cpu().numpy()) <= TOL_ATTN_BF16


@pytest.mark.parametrize("nseq,many_q", [(63, False), (64, False), (100, False), (127, False), (128, False),
                                         (130, False), (100, True)])
def test_forward_many_sequences(dsa, nseq, many_q):
    """Batches of 63 to 130 sequences, decode-like (mostly one query each) or
    prefill-like (8-10 queries each): the kernels locate a row from the batch
    offsets held one per lane below 64 sequences, two per lane from 64 to 127
    and by binary search from 128 on.  Every row against the oracle, and the
    separate calls give the same result bit for bit."""
    announce("forward many sequences", nseq, many_q)
    rng = np.random.default_rng(1000 + nseq)
    ctx = rng.integers(200, 3000, nseq)
    if many_q:
        nq = rng.integers(8, 11, nseq)
    else:
        nq = np.where(rng.random(nseq) < 0.1, rng.integers(2, 6, nseq), 1)
    p = gen.make_problem("fwd", ctx.tolist(), nq.tolist(), H_I=64, H=64, k=512, device=DEV,
                         seed=50 + nseq + int(many_q))
    out, lse, idx = dsa.forward(p)
    idx2 = dsa.topk(p, dsa.indexer_scores(p))
    assert torch.equal(idx, idx2)
    out2, lse2 = dsa.sparse_mla_attn(p, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _check_rows(p, out, idx, np.arange(p.total_q), TOL_ATTN_BF16)

