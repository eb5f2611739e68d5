"""Parity of dsa_topk (HIP) against the CPU oracle: bit-exact on the same scores."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import announce
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_03_amd import dsa as d
    return d


def _problem(seq_ctx, seq_q, k):
    # only the batch layout matters for top-k; keep the other tensors tiny
    return gen.make_problem("topk", seq_ctx, seq_q, H_I=16, d_I=16, H=8, d_qk=16, d_v=16, k=k, device=DEV)


def _run(dsa, p, scores_np, k):
    scores = torch.from_numpy(np.ascontiguousarray(scores_np)).to(DEV)
    got = dsa.topk(p, scores, k=k).cpu().numpy()
    ref = oracle.topk(p.cu_q_host, p.cu_k_host, scores_np, k)
    return got, ref


def _ld(p):
    return (p.max_ctx + 63) // 64 * 64


@pytest.mark.parametrize("k", [1, 32, 100, 2048])
def test_random_scores(dsa, k):
    announce("topk random", k)
    p = _problem([5000, 3000, 20000, 700], [40, 3, 24, 700], k)
    rng = np.random.default_rng(k)
    s = rng.standard_normal((p.total_q, _ld(p))).astype(np.float32)
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


def test_ties_signed_zero_and_nan(dsa):
    announce("topk ties")
    k = 256
    p = _problem([9000, 4096, 300], [16, 16, 16], k)
    rng = np.random.default_rng(5)
    s = rng.integers(-3, 4, (p.total_q, _ld(p))).astype(np.float32)    # heavy ties
    s[s == 0] = np.where(rng.random((s == 0).sum()) < 0.5, -0.0, 0.0)
    s[rng.random(s.shape) < 0.01] = np.nan
    s[3] = 0.5                                                          # all equal
    s[4, ::2] = -0.0
    s[4, 1::2] = 0.0
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


def test_adversarial_orders(dsa):
    """Increasing rows make every chunk overflow the candidate buffer;
    decreasing rows never refill it; both must stay exact."""
    announce("topk monotone rows")
    k = 2048
    p = _problem([40000], [8], k)
    n = _ld(p)
    ramp = np.arange(n, dtype=np.float32)
    s = np.stack([ramp, -ramp, ramp % 7, np.sin(ramp), ramp * 0, (ramp % 4096) - 5, -(ramp % 3), ramp[::-1].copy()])
    got, ref = _run(dsa, p, s.astype(np.float32), k)
    assert np.array_equal(got, ref)


def test_short_rows_select_everything(dsa):
    announce("topk short rows")
    k = 2048
    p = _problem([1024, 2048, 2049, 1], [1024, 1, 2, 1], k)
    s = np.random.default_rng(1).standard_normal((p.total_q, _ld(p))).astype(np.float32)
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, :1], [0]) and np.all(got[0, 1:] == -1)


def test_decode_64x32k_rows(dsa):
    announce("topk decode 64x32k")
    k = 2048
    p = _problem([32768] * 64, [1] * 64, k)
    rng = np.random.default_rng(2)
    s = (0.14 + 0.03 * rng.standard_normal((p.total_q, _ld(p)))).astype(np.float32)   # clustered scores
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("k", [100, 2048])
def test_few_long_rows_use_segments(dsa, k):
    """Few rows: each row is split into segments whose winners are merged."""
    announce("topk segmented", k)
    p = _problem([40000, 3000, 9000, 1000, 70000], [1, 1, 1, 1, 1], k)
    rng = np.random.default_rng(k + 1)
    s = rng.integers(-5, 6, (p.total_q, _ld(p))).astype(np.float32)   # ties across segment borders
    s[4, :] = np.arange(_ld(p), dtype=np.float32) % 977                # periodic: many exact ties
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)
