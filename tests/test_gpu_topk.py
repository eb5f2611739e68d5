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


@pytest.mark.parametrize("k", [1, 100, 2048])
def test_few_rows_radix_select(dsa, k):
    """Few rows: ties, -0/+0, NaN, a row whose keys nearly all fall in one
    histogram bin, keys a few ulps apart.  With k = 2048 every row is shorter
    than 4k entries and takes one radix workgroup (up to 16383 entries, four
    vectors per lane); smaller k split the rows into segments."""
    announce("topk radix", k)
    p = _problem([12000, 16383, 2049, 9000, 500, 15000], [1, 1, 1, 1, 1, 1], k)
    rng = np.random.default_rng(10 + k)
    n = _ld(p)
    s = rng.standard_normal((p.total_q, n)).astype(np.float32)
    s[0] = rng.integers(-3, 4, n).astype(np.float32)                    # heavy ties
    s[0][s[0] == 0] = np.where(rng.random((s[0] == 0).sum()) < 0.5, -0.0, 0.0)
    s[1][rng.random(n) < 0.02] = np.nan
    s[3] = 1.0                                                           # one bin holds almost every key
    s[3, rng.integers(0, 9000, 40)] = rng.standard_normal(40).astype(np.float32)
    s[5] = np.float32(0.25) + np.float32(1e-7) * np.arange(n, dtype=np.float32)        # keys a few ulps apart
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("k", [37, 2048])
def test_long_rows_segments_and_list_merge(dsa, k):
    """Few long rows: each row's segments keep the entries that reach the
    row's sampled threshold and the merge cuts their lists; ties straddle the
    segment borders (2048-entry segments here, 64 per row) and short rows ride
    along."""
    announce("topk segments and list merge", k)
    p = _problem([131072, 2000, 73728, 36865, 100000], [1, 1, 1, 1, 1], k)
    rng = np.random.default_rng(20 + k)
    n = _ld(p)
    s = (0.14 + 0.03 * rng.standard_normal((p.total_q, n))).astype(np.float32)
    s[2] = (np.arange(n) % 1013).astype(np.float32)                     # equal keys in every segment
    s[3] = 0.0
    s[3, 36864] = 1.0                                                    # the best entry is alone in the last segment
    s[4, 50000:] = np.nan
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


def test_very_long_rows_many_segments(dsa):
    """Few very long rows: many segments per row, ties at the cut."""
    announce("topk streaming segments")
    k = 2048
    p = _problem([340000, 5000], [1, 1], k)
    rng = np.random.default_rng(31)
    s = rng.standard_normal((p.total_q, _ld(p))).astype(np.float32)
    s[0, ::3] = 2.5                                                      # ties at the cut
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


def test_segment_threshold_fallbacks(dsa):
    """Few long rows are split into segments that share the row's sampled
    threshold.  A row whose sample blocks hold a few outsized scores gets a
    threshold that fewer than k entries reach, so the merge must select that
    row again without it; a row of small integers puts so many ties on the
    threshold that the segments' lists overflow the merge's buffer; a row of
    exactly the sample's size is sampled whole, one entry shorter not at all."""
    announce("topk segment fallbacks")
    k = 2048
    ctx = [60000, 131072, 20000, 4096, 5000, 4095]
    p = _problem(ctx, [1] * len(ctx), k)
    rng = np.random.default_rng(60)
    s = (0.14 + 0.03 * rng.standard_normal((p.total_q, _ld(p)))).astype(np.float32)
    n = ctx[0]
    rank = min(4096, 13 * k * 4096 // (10 * n) + 8)
    for b in range(4):
        start = (b * (n - 1024) // 3) & ~3
        s[0, start:start + rank // 4 + 1] = 100.0                      # the sample's top ranks: too high
    s[1] = rng.integers(-2, 3, _ld(p)).astype(np.float32)
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


def test_segment_cut_inside_a_segment(dsa):
    """40 rows of 131072 entries take segments of 10240 entries (13 per row
    on 256 CUs).  A hot region of 10240 entries between the sample blocks
    puts every entry of its segment above the row's threshold, so that
    segment's buffer overflows and is cut to its k best while streaming; in
    one row the hot entries all tie (the earliest k win), in another they
    straddle two segments."""
    announce("topk segment cut inside a segment")
    k = 2048
    p = _problem([131072] * 40, [1] * 40, k)
    rng = np.random.default_rng(70)
    s = (0.14 + 0.03 * rng.standard_normal((p.total_q, _ld(p)))).astype(np.float32)
    s[3, 20480:30720] = (10.0 + rng.standard_normal(10240)).astype(np.float32)
    s[7, 20480:30720] = 10.0                                             # ties: the earliest k win
    s[11, 25000:35240] = (10.0 + rng.standard_normal(10240)).astype(np.float32)
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("k", [5, 2048])
def test_few_short_rows_one_radix_pass(dsa, k):
    """Few rows too short to split: one radix workgroup per row, no workspace."""
    announce("topk radix unsplit", k)
    p = _problem([6000, 3000, 7000, 2048], [1, 1, 1, 2], k)
    rng = np.random.default_rng(40 + k)
    s = rng.standard_normal((p.total_q, _ld(p))).astype(np.float32)
    s[1] = np.round(s[1])                                                # ties
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


def test_long_rows_sampled_threshold(dsa):
    """Rows of 16K candidates or more start from a threshold sampled from four
    blocks of 1024 entries spread over the row.  Rows whose blocks hold a few
    outsized scores make the sample overestimate it (fewer than k entries reach
    it), and those rows must fall back to the plain pass; integer rows put
    many ties on the sampled threshold."""
    announce("topk sampled threshold")
    k = 2048
    p = _problem([40000], [300], k)
    rng = np.random.default_rng(50)
    n_ld = _ld(p)
    s = (0.14 + 0.03 * rng.standard_normal((p.total_q, n_ld))).astype(np.float32)
    s[1::3] = rng.integers(-2, 3, (len(s[1::3]), n_ld)).astype(np.float32)
    for r in range(0, p.total_q, 3):
        n = 40000 - p.total_q + r + 1
        rank = min(4096, 13 * k * 4096 // (10 * n) + 8)
        for b in range(4):
            start = (b * (n - 1024) // 3) & ~3
            s[r, start:start + rank // 4 + 1] = 100.0                  # the sample's top ranks: too high
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("k", [512, 2048])
def test_special_values_on_the_threshold(dsa, k):
    """Scores drawn from a few special floats (both infinities, the largest
    finite and smallest normal magnitudes, denormals, both zeros, NaN) in
    per-row mixtures, so that the k-th key and the running thresholds land on
    them.  The prefill filter compares floats against the smallest float above
    each threshold key; it must admit exactly the keys above it, on the short
    rows' plain stream and on the long rows' sampled threshold alike."""
    announce("topk special values", k)
    p = _problem([20000, 6000, 40000], [8, 8, 8], k)
    rng = np.random.default_rng(77 + k)
    vals = np.array([-np.inf, -3.4e38, -1.0, -1e-45, -0.0, 0.0, 1e-45, 3e-45, 1.1754944e-38, 1.0, 3.4e38,
                     np.inf, np.nan], dtype=np.float32)
    s = np.empty((p.total_q, _ld(p)), np.float32)
    for r in range(p.total_q):
        w = rng.dirichlet(np.full(len(vals), 0.3))
        s[r] = vals[rng.choice(len(vals), size=s.shape[1], p=w)]
    # a few rows with fewer than k entries above -inf or above NaN
    s[2] = np.where(rng.random(s.shape[1]) < 0.005, 1.0, -np.inf)
    s[10] = np.where(rng.random(s.shape[1]) < 0.005, 0.0, np.nan)
    s[17] = np.where(rng.random(s.shape[1]) < 0.5, 1e-45, -0.0)
    got, ref = _run(dsa, p, s, k)
    assert np.array_equal(got, ref)
