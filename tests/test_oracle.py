"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something other than itself: a library
routine (numpy matmul / lexsort, torch's fp8 decoding, torch's scaled-dot-
product attention), a closed form, an invariant, or brute force on tiny
inputs.  Mistakes these are built to catch: a dropped weight or head, a wrong
sign in the activation, a transposed operand, a wrong key row or causal bound,
a wrong tie rule, a wrong value slice or softmax scale.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_03_amd import inputs as gen


def _ragged(seq_ctx, seq_q):
    cu_q = np.concatenate([[0], np.cumsum(seq_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(seq_ctx)]).astype(np.int32)
    return cu_q, cu_k


def _positions(cu_q, cu_k):
    pos, base = [], []
    for b in range(len(cu_q) - 1):
        qb, ctx = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for r in range(qb):
            pos.append(ctx - qb + r)
            base.append(cu_k[b])
    return np.array(pos), np.array(base)


# ---------------------------------------------------------------- formats

def test_e4m3_table_matches_torch_decoding():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # spot values of the OCP E4M3FN definition
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x38) == 1.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) == -1.0


def test_bf16_and_fp8_storage_decode_like_fp32():
    """The same values stored as bf16 / e4m3 / fp32 give identical results."""
    g = torch.Generator().manual_seed(3)
    vals = torch.randint(-4, 5, (40, 2, 16), generator=g).to(torch.float32)
    keys = torch.randint(-4, 5, (40, 16), generator=g).to(torch.float32)
    w = torch.rand(40, 2, generator=g)
    cu_q, cu_k = _ragged([40], [40])
    s32 = oracle.indexer(cu_q, cu_k, vals.numpy(), keys.numpy(), w.numpy())
    s8 = oracle.indexer(cu_q, cu_k, gen.storage_numpy(vals.to(torch.float8_e4m3fn)),
                        gen.storage_numpy(keys.to(torch.float8_e4m3fn)), w.numpy())
    assert np.array_equal(s32, s8)
    q = torch.randn(40, 3, 16, generator=g).to(torch.bfloat16)
    kv = torch.randn(40, 16, generator=g).to(torch.bfloat16)
    idx = np.tile(np.arange(8, dtype=np.int32), (40, 1))
    idx[:8] = -1
    for r in range(8):
        idx[r, :r + 1] = np.arange(r + 1)
    o16, l16 = oracle.sparse_mla(cu_q, cu_k, gen.storage_numpy(q), gen.storage_numpy(kv), idx, 8, 0.3)
    o32, l32 = oracle.sparse_mla(cu_q, cu_k, q.float().numpy(), kv.float().numpy(), idx, 8, 0.3)
    assert np.array_equal(o16, o32) and np.array_equal(l16, l32)


# ---------------------------------------------------------------- indexer

def _indexer_case(seed, seq_ctx, seq_q, H_I, d_I, integer=False):
    rng = np.random.default_rng(seed)
    cu_q, cu_k = _ragged(seq_ctx, seq_q)
    T, K = cu_q[-1], cu_k[-1]
    if integer:
        q = rng.integers(-4, 5, (T, H_I, d_I)).astype(np.float32)
        k = rng.integers(-4, 5, (K, d_I)).astype(np.float32)
        w = (rng.integers(0, 9, (T, H_I)) * 0.25).astype(np.float32)
    else:
        q = rng.standard_normal((T, H_I, d_I)).astype(np.float32)
        k = rng.standard_normal((K, d_I)).astype(np.float32)
        w = rng.uniform(-1, 1, (T, H_I)).astype(np.float32)
    return cu_q, cu_k, q, k, w


@pytest.mark.parametrize("act", [oracle.ACT_RELU, oracle.ACT_GELU])
@pytest.mark.parametrize("integer", [False, True])
def test_indexer_antisymmetric_part_is_a_matmul(act, integer):
    """relu(x) - relu(-x) = x and gelu(x) - gelu(-x) = x, so
    I(q) - I(-q) = sum_j w_j q_j . k_s = ((w q) summed over heads) @ k^T."""
    cu_q, cu_k, q, k, w = _indexer_case(1, [37, 50, 9], [37, 4, 1], 3, 8, integer)
    ld = 50
    plus = oracle.indexer(cu_q, cu_k, q, k, w, act=act, ld=ld)
    minus = oracle.indexer(cu_q, cu_k, -q, k, w, act=act, ld=ld)
    pos, base = _positions(cu_q, cu_k)
    wq = np.einsum("tj,tjd->td", w.astype(np.float64), q.astype(np.float64))
    for i in range(len(pos)):
        keys = k[base[i]: base[i] + pos[i] + 1].astype(np.float64)
        want = keys @ wq[i]
        got = plus[i, :pos[i] + 1] - minus[i, :pos[i] + 1]
        if integer and act == oracle.ACT_RELU:
            assert np.array_equal(got, want)
        else:
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
        assert np.all(plus[i, pos[i] + 1:] == 0.0)  # beyond the causal bound: untouched


def test_indexer_relu_symmetric_part_is_abs():
    """relu(x) + relu(-x) = |x|: I(q) + I(-q) = sum_j w_j |q_j . k_s|; with w >= 0
    every score is >= 0 and a row whose dot products are all <= 0 scores 0."""
    cu_q, cu_k, q, k, w = _indexer_case(2, [64], [64], 4, 16, integer=True)
    w = np.abs(w)
    plus = oracle.indexer(cu_q, cu_k, q, k, w)
    minus = oracle.indexer(cu_q, cu_k, -q, k, w)
    dots = np.einsum("tjd,sd->tjs", q.astype(np.float64), k.astype(np.float64))
    want = np.einsum("tj,tjs->ts", w.astype(np.float64), np.abs(dots))
    mask = np.tril(np.ones((64, 64), dtype=bool))
    assert np.array_equal((plus + minus)[mask], want[mask])
    assert np.all(plus >= 0.0)
    # all dot products negative -> zero score
    qq = -np.abs(q)
    kk = np.abs(k)
    assert np.all(oracle.indexer(cu_q, cu_k, qq, kk, w)[mask] == 0.0)


def test_indexer_gelu_value_is_x_times_normal_cdf():
    from scipy.stats import norm
    xs = np.array([-2.5, -1.0, -0.3, 0.0, 0.7, 1.0, 3.0], dtype=np.float32)
    n = len(xs)
    cu_q, cu_k = _ragged([n], [n])
    q = np.ones((n, 1, 1), dtype=np.float32)
    k = xs.reshape(n, 1)
    w = np.ones((n, 1), dtype=np.float32)
    got = oracle.indexer(cu_q, cu_k, q, k, w, act=oracle.ACT_GELU)
    want = xs.astype(np.float64) * norm.cdf(xs.astype(np.float64))
    assert abs(got[n - 1, 5] - 0.8413447460685429) < 1e-15   # GELU(1) = Phi(1)
    for s in range(n):
        assert abs(got[n - 1, s] - want[s]) < 1e-14


def test_indexer_heads_are_weighted_independently():
    """w = e_j isolates head j: the score is relu(q_j . k_s)."""
    cu_q, cu_k, q, k, _ = _indexer_case(5, [20], [20], 3, 4, integer=True)
    for j in range(3):
        w = np.zeros((20, 3), dtype=np.float32)
        w[:, j] = 1.0
        got = oracle.indexer(cu_q, cu_k, q, k, w)
        dots = q[:, j, :].astype(np.float64) @ k.T.astype(np.float64)
        want = np.where(np.tril(np.ones((20, 20), bool)), np.maximum(dots, 0.0), 0.0)
        assert np.array_equal(got, want)


# ---------------------------------------------------------------- top-k

def _brute_force_topk(scores, n, k):
    """The unique k-subset S with: for s in S, u not in S: s beats u."""
    def beats(a, b):
        sa, sb = scores[a], scores[b]
        if np.isnan(sa) or np.isnan(sb):
            if np.isnan(sa) and np.isnan(sb):
                return a < b
            return np.isnan(sb)
        return sa > sb or (sa == sb and a < b)
    found = []
    for S in itertools.combinations(range(n), k):
        rest = [u for u in range(n) if u not in S]
        if all(beats(s, u) for s in S for u in rest):
            found.append(list(S))
    assert len(found) == 1
    return found[0]


def test_topk_matches_subset_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 6))
        vals = rng.integers(-3, 4, n).astype(np.float32)   # many ties
        if trial % 5 == 0:
            vals[rng.integers(0, n)] = np.nan
        if trial % 3 == 0:
            vals[vals == 0] = -0.0
        cu_q, cu_k = _ragged([n], [1])
        got = oracle.topk(cu_q, cu_k, vals.reshape(1, n), k)[0]
        if n <= k:
            want = list(range(n)) + [-1] * (k - n)
        else:
            want = _brute_force_topk(vals, n, k)
        assert list(got) == want, (vals, k)


def test_topk_matches_lexsort_on_ragged_rows():
    rng = np.random.default_rng(8)
    cu_q, cu_k = _ragged([300, 17, 129], [300, 5, 2])
    pos, _ = _positions(cu_q, cu_k)
    ld = 300
    scores = rng.integers(0, 50, (len(pos), ld)).astype(np.float32)   # ties everywhere
    k = 32
    got = oracle.topk(cu_q, cu_k, scores, k)
    for i, p in enumerate(pos):
        n = p + 1
        row = scores[i, :n]
        order = np.lexsort((np.arange(n), -row))    # score desc, then position asc
        want = np.sort(order[:k]) if n > k else np.arange(n)
        want = np.concatenate([want, -np.ones(k - len(want), np.int64)])
        assert np.array_equal(got[i], want)


def test_topk_invariants():
    rng = np.random.default_rng(9)
    n, k = 500, 64
    cu_q, cu_k = _ragged([n], [1])
    row = rng.standard_normal(n).astype(np.float32)
    base = oracle.topk(cu_q, cu_k, row.reshape(1, n), k)[0]
    # strictly increasing transform: same selection
    mono = (np.exp(row.astype(np.float64)) * 3.0 + 1.0).astype(np.float32)
    assert np.array_equal(oracle.topk(cu_q, cu_k, mono.reshape(1, n), k)[0], base)
    # permuting positions maps the selection (distinct scores)
    perm = rng.permutation(n)
    permuted = np.empty_like(row)
    permuted[perm] = row
    sel = oracle.topk(cu_q, cu_k, permuted.reshape(1, n), k)[0]
    assert np.array_equal(np.sort(perm[base]), sel)
    # all-equal row: the first k positions
    assert np.array_equal(oracle.topk(cu_q, cu_k, np.full((1, n), 0.5, np.float32), k)[0], np.arange(k))
    # -0 and +0 tie: lower index wins
    z = np.zeros((1, n), np.float32)
    z[0, ::2] = -0.0
    assert np.array_equal(oracle.topk(cu_q, cu_k, z, k)[0], np.arange(k))


# ---------------------------------------------------------------- attention

def _dense_causal_mqa_torch(q, kv, d_v, scale):
    """Library reference: torch SDPA in float64, causal, all heads sharing the
    one latent as key (all columns) and value (first d_v columns)."""
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)         # [H, L, d]
    k = torch.from_numpy(kv.astype(np.float64)).unsqueeze(0).expand(q.shape[1], -1, -1)
    v = torch.from_numpy(kv[:, :d_v].astype(np.float64)).unsqueeze(0).expand(q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attention_with_all_candidates_equals_dense_causal_mqa():
    rng = np.random.default_rng(11)
    L, H, d_qk, d_v, k = 48, 4, 24, 16, 64     # k >= L: every candidate selected
    q = rng.standard_normal((L, H, d_qk)).astype(np.float32)
    kv = rng.standard_normal((L, d_qk)).astype(np.float32)
    cu_q, cu_k = _ragged([L], [L])
    idx = oracle.topk(cu_q, cu_k, rng.standard_normal((L, L)).astype(np.float32), k)
    scale = 0.37
    out, lse = oracle.sparse_mla(cu_q, cu_k, q, kv, idx, d_v, scale)
    ref = _dense_causal_mqa_torch(q, kv, d_v, scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # lse from a library logsumexp
    logits = scale * np.einsum("thd,sd->ths", q.astype(np.float64), kv.astype(np.float64))
    mask = np.tril(np.ones((L, L), bool))[:, None, :]
    ref_lse = torch.logsumexp(torch.from_numpy(np.where(mask, logits, -np.inf)), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(12)
    L, H, d_qk, d_v = 30, 3, 10, 6
    q = rng.standard_normal((L, H, d_qk)).astype(np.float32)
    kv = rng.standard_normal((L, d_qk)).astype(np.float32)
    cu_q, cu_k = _ragged([L], [L])
    # one selected entry: o = v_s exactly, lse = z_s
    idx = -np.ones((L, 4), np.int32)
    idx[:, 0] = np.arange(L) // 2
    out, lse = oracle.sparse_mla(cu_q, cu_k, q, kv, idx, d_v, 0.5)
    for t in range(L):
        s = t // 2
        assert np.array_equal(out[t], np.tile(kv[s, :d_v].astype(np.float64), (H, 1)))
        z = 0.5 * (q[t].astype(np.float64) @ kv[s].astype(np.float64))
        np.testing.assert_allclose(lse[t], z, rtol=0, atol=1e-13)
    # q = 0: mean of the selected value rows, lse = log(count)
    idx = np.tile(np.array([0, 3, 7, -1], np.int32), (L, 1))
    idx[:8] = np.array([0, -1, -1, -1])
    out, lse = oracle.sparse_mla(cu_q, cu_k, np.zeros_like(q), kv, idx, d_v, 0.5)
    mean = kv[[0, 3, 7], :d_v].astype(np.float64).mean(0)
    np.testing.assert_allclose(out[10], np.tile(mean, (H, 1)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[10], np.log(3.0), rtol=0, atol=1e-14)
    # two entries: o = sigmoid(z1 - z2) v1 + sigmoid(z2 - z1) v2
    idx = np.tile(np.array([1, 4], np.int32), (L, 1))
    idx[:5] = np.array([0, -1])
    out, _ = oracle.sparse_mla(cu_q, cu_k, q, kv, idx, d_v, 0.9)
    t = 20
    z = 0.9 * (q[t].astype(np.float64) @ kv[[1, 4]].astype(np.float64).T)   # [H, 2]
    sig = 1.0 / (1.0 + np.exp(-(z[:, 0] - z[:, 1])))
    want = sig[:, None] * kv[1, :d_v] + (1 - sig)[:, None] * kv[4, :d_v]
    np.testing.assert_allclose(out[t], want, rtol=0, atol=1e-13)
    # empty selection
    idx = -np.ones((L, 4), np.int32)
    out, lse = oracle.sparse_mla(cu_q, cu_k, q, kv, idx, d_v, 0.5)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


def test_attention_invariants():
    rng = np.random.default_rng(13)
    L, H, d_qk, d_v, k = 64, 4, 16, 8, 12
    q = rng.standard_normal((L, H, d_qk)).astype(np.float32)
    kv = rng.standard_normal((L, d_qk)).astype(np.float32)
    cu_q, cu_k = _ragged([L], [L])
    idx = oracle.topk(cu_q, cu_k, rng.standard_normal((L, L)).astype(np.float32), k)
    out, lse = oracle.sparse_mla(cu_q, cu_k, q, kv, idx, d_v, 0.25)
    # order of the index list is irrelevant
    perm_idx = idx[:, rng.permutation(k)]
    out2, lse2 = oracle.sparse_mla(cu_q, cu_k, q, kv, perm_idx, d_v, 0.25)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    # rows that no query selected are irrelevant
    used = np.zeros(L, bool)
    used[idx[idx >= 0]] = True
    garbage = kv.copy()
    garbage[~used] = 1e6
    out3, lse3 = oracle.sparse_mla(cu_q, cu_k, q, garbage, idx, d_v, 0.25)
    assert np.array_equal(out3, out) and np.array_equal(lse3, lse)
    # heads with identical queries give identical outputs
    q4 = q.copy()
    q4[:, 1] = q4[:, 0]
    out4, _ = oracle.sparse_mla(cu_q, cu_k, q4, kv, idx, d_v, 0.25)
    assert np.array_equal(out4[:, 0], out4[:, 1])


# ------------------------------------------------- dense (masked mode) attention

def test_dense_attention_equals_masked_sdpa_on_ragged_batches():
    """Dense causal MQA: every query row attends to all of [0, pos].  Checked
    against torch SDPA in float64 with the causal mask written out, per
    sequence: a prefill sequence, a decode-like one (3 queries at the end of 50
    cached tokens) and a one-token sequence."""
    rng = np.random.default_rng(21)
    ctx, nq, H, d_qk, d_v = [40, 50, 1], [40, 3, 1], 3, 12, 8
    cu_q, cu_k = _ragged(ctx, nq)
    q = rng.standard_normal((sum(nq), H, d_qk)).astype(np.float32)
    kv = rng.standard_normal((sum(ctx), d_qk)).astype(np.float32)
    out, lse = oracle.dense_mla(cu_q, cu_k, q, kv, d_v, 0.31)
    for b in range(len(ctx)):
        qb = q[cu_q[b]:cu_q[b + 1]].astype(np.float64)
        kb = kv[cu_k[b]:cu_k[b + 1]].astype(np.float64)
        pos = ctx[b] - nq[b] + np.arange(nq[b])
        mask = np.arange(ctx[b])[None, :] <= pos[:, None]                  # [nq, ctx]
        qt = torch.from_numpy(qb).permute(1, 0, 2)
        k = torch.from_numpy(kb).unsqueeze(0).expand(H, -1, -1)
        v = torch.from_numpy(kb[:, :d_v].copy()).unsqueeze(0).expand(H, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=torch.from_numpy(mask),
                                                               scale=0.31).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[cu_q[b]:cu_q[b + 1]], ref, rtol=0, atol=1e-12)
        logits = 0.31 * np.einsum("thd,sd->ths", qb, kb)
        ref_lse = torch.logsumexp(torch.from_numpy(np.where(mask[:, None, :], logits, -np.inf)), dim=-1).numpy()
        np.testing.assert_allclose(lse[cu_q[b]:cu_q[b + 1]], ref_lse, rtol=0, atol=1e-12)


def test_dense_attention_closed_forms_and_causality():
    rng = np.random.default_rng(22)
    L, H, d_qk, d_v = 20, 2, 6, 4
    cu_q, cu_k = _ragged([L], [L])
    q = rng.standard_normal((L, H, d_qk)).astype(np.float32)
    kv = rng.standard_normal((L, d_qk)).astype(np.float32)
    # q = 0: the mean of v over [0, pos], lse = log(pos + 1)
    out, lse = oracle.dense_mla(cu_q, cu_k, np.zeros_like(q), kv, d_v, 0.7)
    for t in range(L):
        np.testing.assert_allclose(out[t], np.tile(kv[:t + 1, :d_v].astype(np.float64).mean(0), (H, 1)),
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[t], np.log(t + 1.0), rtol=0, atol=1e-14)
    # position 0 sees itself only
    out, lse = oracle.dense_mla(cu_q, cu_k, q, kv, d_v, 0.7)
    assert np.array_equal(out[0], np.tile(kv[0, :d_v].astype(np.float64), (H, 1)))
    # future rows never matter
    for t in (3, 11):
        late = kv.copy()
        late[t + 1:] = 1e6
        o2, l2 = oracle.dense_mla(cu_q, cu_k, q, late, d_v, 0.7)
        assert np.array_equal(o2[:t + 1], out[:t + 1]) and np.array_equal(l2[:t + 1], lse[:t + 1])


# ------------------------------------------------------ indexer-key quantisation

def _e4m3_values():
    return np.array([oracle.e4m3_value(c) for c in range(256)])


def test_quantize_every_code_round_trips_and_ties_go_even():
    vals = _e4m3_values()
    finite = [c for c in range(256) if np.isfinite(vals[c])]
    x = np.array([vals[c] for c in finite], np.float32)[None, :]
    codes = oracle.quantize_keys(x)[0]
    want = np.array(finite, np.uint8)
    assert np.array_equal(codes, want)                      # every finite code, -0 included
    # midpoints between neighbouring positive values go to the even code,
    # points just beside them to the nearer one
    pos = np.array([vals[c] for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2
    codes_mid = oracle.quantize_keys(mids.astype(np.float32)[None, :])[0]
    even = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(codes_mid, even.astype(np.uint8))
    below = oracle.quantize_keys(np.nextafter(mids.astype(np.float32), np.float32(0))[None, :])[0]
    above = oracle.quantize_keys(np.nextafter(mids.astype(np.float32), np.float32(1e9))[None, :])[0]
    assert np.array_equal(below, np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(above, np.arange(1, 0x7F, dtype=np.uint8))


def test_quantize_saturation_nan_and_library_rounding():
    x = np.array([[448.0, 449.0, 464.0, 1e30, -500.0, np.nan, -0.0, 1e-30, -1e-30]], np.float32)
    codes = oracle.quantize_keys(x)[0]
    assert list(codes) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80, 0x00, 0x80]
    # in range, torch's conversion (round to nearest even) gives the same codes
    rng = np.random.default_rng(31)
    y = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 5, (64, 1)))).astype(np.float32)
    y = np.clip(y, -440, 440)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quantize_keys(y), ref)
    # bfloat16 sources decode exactly first
    bits = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref_b = torch.from_numpy(y).to(torch.bfloat16).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quantize_keys(bits), ref_b)


def test_quantize_per_token_scale():
    vals = _e4m3_values()
    rng = np.random.default_rng(32)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    x[0] *= 1e-3
    x[1] *= 1e3
    x[2] = 0.0
    x[3, :] = 0.5
    x[3, 7] = 448.0 * 4.0            # amax exactly 448 * 2^2: e = 2
    x[4, :] = 0.5
    x[4, 9] = np.nextafter(np.float32(448.0 * 4.0), np.float32(1e9))  # just above: e = 3
    codes, sc = oracle.quantize_keys(x, scaled=True)
    # an infinity takes the largest scale; NaN takes no part in the maximum
    y = np.array([[1.0, -np.inf, 2.0, np.nan], [np.nan, 448.0, -3.0, 1.0]], np.float32)
    cy, sy = oracle.quantize_keys(y, scaled=True)
    assert list(sy) == [127 + 127, 127] and list(cy[1]) == [0x7F, 0x7E, 0xC4, 0x38]
    assert cy[0, 1] == 0xFE and cy[0, 3] == 0x7F and cy[0, 0] == 0x00
    e = sc.astype(np.int64) - 127
    assert e[2] == 0 and np.all(codes[2] == 0)
    assert e[3] == 2 and codes[3, 7] == 0x7E
    assert e[4] == 3
    for t in range(6):
        amax = np.abs(x[t]).max()
        if amax > 0:
            assert amax <= 448.0 * 2.0 ** e[t] and amax > 448.0 * 2.0 ** (e[t] - 1)
        deq = vals[codes[t]] * 2.0 ** e[t]
        # the scaled codes are the unscaled quantisation of x / 2^e
        assert np.array_equal(codes[t], oracle.quantize_keys((x[t] / np.float32(2.0 ** e[t]))[None, :])[0])
        # relative error of normal values at most 2^-4 (3 mantissa bits, round to nearest)
        big = np.abs(x[t]) >= 2.0 ** (e[t] - 6)
        assert np.all(np.abs(deq[big] - x[t][big]) <= np.abs(x[t][big]) * 2.0 ** -4)


def _fp8_keys_case(seed, n, d):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    return codes


@pytest.mark.parametrize("act", [oracle.ACT_RELU, oracle.ACT_GELU])
def test_scaled_fp8_keys_equal_their_dequantised_values(act):
    """A key with E8M0 byte b is value(code) * 2^(b - 127): the scores of scaled
    FP8 keys equal those of float32 keys holding exactly those values."""
    vals = _e4m3_values()
    cu_q, cu_k = _ragged([40, 23], [40, 5])
    rng = np.random.default_rng(33)
    kc = _fp8_keys_case(33, 63, 32)
    qc = _fp8_keys_case(34, 45, 2 * 32).reshape(45, 2, 32)
    sc = rng.integers(127 - 12, 127 + 12, 63).astype(np.uint8)
    w = rng.standard_normal((45, 2)).astype(np.float32)
    got = oracle.indexer(cu_q, cu_k, qc, kc, w, act=act, k_scale=sc)
    kf = (vals[kc] * 2.0 ** (sc.astype(np.int64) - 127)[:, None]).astype(np.float32)
    assert np.array_equal(kf.astype(np.float64), vals[kc] * 2.0 ** (sc.astype(np.int64) - 127)[:, None])
    want = oracle.indexer(cu_q, cu_k, vals[qc].astype(np.float32), kf, w, act=act)
    assert np.array_equal(got, want)
    # scale byte 127 is the unscaled key
    same = oracle.indexer(cu_q, cu_k, qc, kc, w, act=act, k_scale=np.full(63, 127, np.uint8))
    assert np.array_equal(same, oracle.indexer(cu_q, cu_k, qc, kc, w, act=act))


def test_relu_scores_are_homogeneous_in_the_key_scale():
    """ReLU(2^e x) = 2^e ReLU(x): one scale for every key multiplies each score."""
    cu_q, cu_k = _ragged([30], [30])
    kc = _fp8_keys_case(35, 30, 16)
    qc = _fp8_keys_case(36, 30, 3 * 16).reshape(30, 3, 16)
    w = np.random.default_rng(36).standard_normal((30, 3)).astype(np.float32)
    base = oracle.indexer(cu_q, cu_k, qc, kc, w)
    for e in (-20, -1, 3, 17):
        got = oracle.indexer(cu_q, cu_k, qc, kc, w, k_scale=np.full(30, 127 + e, np.uint8))
        assert np.array_equal(got, base * 2.0 ** e)


# ------------------------------------------------------ indexer alignment loss

def _target_case(seed, seq_ctx, seq_q, H, d):
    rng = np.random.default_rng(seed)
    cu_q, cu_k = _ragged(seq_ctx, seq_q)
    q = (rng.standard_normal((int(cu_q[-1]), H, d)) * 0.7).astype(np.float32)
    kv = rng.standard_normal((int(cu_k[-1]), d)).astype(np.float32)
    return cu_q, cu_k, q, kv


def test_attn_target_dense_is_the_head_mean_of_softmax():
    """Summing the heads' softmax rows and L1-normalising is the head mean of
    torch's softmax over the causal candidates."""
    cu_q, cu_k, q, kv = _target_case(60, [37, 50, 9], [37, 4, 1], 3, 16)
    scale = 0.3
    p = oracle.attn_target(cu_q, cu_k, q, kv, scale)
    pos, base = _positions(cu_q, cu_k)
    assert p.shape == (len(pos), 50)
    for i in range(len(pos)):
        n = pos[i] + 1
        z = scale * torch.from_numpy(q[i]).double() @ torch.from_numpy(kv[base[i]: base[i] + n]).double().T
        want = torch.softmax(z, dim=-1).mean(0).numpy()
        np.testing.assert_allclose(p[i, :n], want, rtol=1e-12, atol=1e-15)
        assert np.all(p[i, n:] == 0.0)
        assert abs(p[i].sum() - 1.0) < 1e-12


def test_attn_target_over_a_selected_set():
    cu_q, cu_k, q, kv = _target_case(61, [40, 33], [40, 2], 2, 8)
    scale = 0.5
    pos, base = _positions(cu_q, cu_k)
    rng = np.random.default_rng(62)
    k = 12
    idx = np.full((len(pos), k), -1, np.int32)
    for i in range(len(pos)):
        n = pos[i] + 1
        sel = np.sort(rng.choice(n, min(n, k), replace=False)) if n > k else np.arange(n)
        idx[i, :len(sel)] = sel
    p = oracle.attn_target(cu_q, cu_k, q, kv, scale, idx=idx)
    for i in range(len(pos)):
        sel = idx[i][idx[i] >= 0]
        z = scale * torch.from_numpy(q[i]).double() @ torch.from_numpy(kv[base[i] + sel]).double().T
        want = torch.softmax(z, dim=-1).mean(0).numpy()
        np.testing.assert_allclose(p[i, :len(sel)], want, rtol=1e-12, atol=1e-15)
        assert np.all(p[i, len(sel):] == 0.0)
    # selecting every candidate is the dense target
    cu_q2, cu_k2, q2, kv2 = _target_case(63, [20], [20], 3, 8)
    all_idx = np.where(np.arange(20)[None, :] <= np.arange(20)[:, None], np.arange(20)[None, :], -1).astype(np.int32)
    np.testing.assert_allclose(oracle.attn_target(cu_q2, cu_k2, q2, kv2, 0.4, idx=all_idx),
                               oracle.attn_target(cu_q2, cu_k2, q2, kv2, 0.4), rtol=0, atol=1e-15)


def test_indexer_kl_matches_torch_autograd():
    rng = np.random.default_rng(64)
    nrows, m = 9, 30
    cnt = np.array([30, 1, 5, 17, 0, 29, 2, 30, 11], np.int32)
    I = rng.standard_normal((nrows, m)) * 3
    p = rng.random((nrows, m)) ** 3
    p[:, ::4] = 0.0                                       # zero targets: 0 log 0 = 0
    for i in range(nrows):
        p[i, cnt[i]:] = 0.0
        if p[i].sum() > 0:
            p[i] /= p[i].sum()
    loss, dI = oracle.indexer_kl(I, p, cnt)
    for i in range(nrows):
        n = cnt[i]
        if n == 0:
            assert loss[i] == 0.0 and np.all(dI[i] == 0.0)
            continue
        Iv = torch.tensor(I[i, :n], dtype=torch.float64, requires_grad=True)
        pv = torch.tensor(p[i, :n], dtype=torch.float64)
        ref = torch.nn.functional.kl_div(torch.log_softmax(Iv, 0), pv, reduction="sum")
        ref.backward()
        assert abs(loss[i] - ref.item()) <= 1e-12 * max(1.0, abs(ref.item()))
        np.testing.assert_allclose(dI[i, :n], Iv.grad.numpy(), rtol=1e-11, atol=1e-14)
        assert np.all(dI[i, n:] == 0.0)
    # closed forms: p = softmax(I) gives 0 and no gradient; a one-hot p gives -log softmax(I)_e
    row = rng.standard_normal(7)
    sm = np.exp(row - row.max()) / np.exp(row - row.max()).sum()
    l0, g0 = oracle.indexer_kl(row[None, :], sm[None, :], [7])
    assert abs(l0[0]) < 1e-15 and np.max(np.abs(g0)) < 1e-15
    onehot = np.zeros(7)
    onehot[3] = 1.0
    l1, g1 = oracle.indexer_kl(row[None, :], onehot[None, :], [7])
    assert abs(l1[0] + np.log(sm[3])) < 1e-13
    np.testing.assert_allclose(g1[0], sm - onehot, atol=1e-15)


def _torch_index_grads(cu_q, cu_k, q_idx, k_idx, w, g, act, idx=None):
    """Gradients of sum_i sum_e g[i, e] I[i, s_e] through torch's autograd, the
    index score built from torch ops in float64."""
    pos, base = _positions(cu_q, cu_k)
    qt = torch.tensor(q_idx, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k_idx, dtype=torch.float64, requires_grad=True)
    total = torch.zeros((), dtype=torch.float64)
    for i in range(len(pos)):
        if idx is None:
            sel = np.arange(pos[i] + 1)
            gi = g[i, :pos[i] + 1]
        else:
            keep = idx[i] >= 0
            sel = idx[i][keep]
            gi = g[i][keep]
        x = qt[i] @ kt[torch.from_numpy(base[i] + sel)].T
        a = torch.relu(x) if act == oracle.ACT_RELU else torch.nn.functional.gelu(x)
        total = total + (torch.from_numpy(gi) * (wt[i] @ a)).sum()
    total.backward()
    return qt.grad.numpy(), wt.grad.numpy(), kt.grad.numpy()


@pytest.mark.parametrize("act,integer", [(oracle.ACT_RELU, True), (oracle.ACT_RELU, False), (oracle.ACT_GELU, False)])
def test_indexer_backward_matches_torch_autograd(act, integer):
    cu_q, cu_k, q, k, w = _indexer_case(65, [23, 30], [23, 3], 3, 8, integer)
    pos, _ = _positions(cu_q, cu_k)
    rng = np.random.default_rng(66)
    g = rng.standard_normal((len(pos), 30))
    for i in range(len(pos)):
        g[i, pos[i] + 1:] = 0.0
    dq, dw, dk = oracle.indexer_backward(cu_q, cu_k, q, k, w, g, act=act)
    rq, rw, rk = _torch_index_grads(cu_q, cu_k, q, k, w, g, act)
    for got, ref in ((dq, rq), (dw, rw), (dk, rk)):
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)
    if integer:
        # integer inputs put many dot products exactly at 0, where both take ReLU's slope as 0
        assert np.any(np.einsum("tjd,sd->tjs", q, k) == 0)
    # over a selected set (ascending, -1 padded)
    m = 6
    idx = np.full((len(pos), m), -1, np.int32)
    for i in range(len(pos)):
        n = pos[i] + 1
        sel = np.sort(rng.choice(n, min(n, m), replace=False))
        idx[i, :len(sel)] = sel
    gs = rng.standard_normal((len(pos), m))
    dq, dw, dk = oracle.indexer_backward(cu_q, cu_k, q, k, w, gs, act=act, idx=idx)
    rq, rw, rk = _torch_index_grads(cu_q, cu_k, q, k, w, gs, act, idx=idx)
    for got, ref in ((dq, rq), (dw, rw), (dk, rk)):
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_indexer_backward_with_key_scales():
    """FP8 codes with per-token scales give the gradients of float32 keys
    holding the dequantised values (dk with respect to the dequantised key)."""
    vals = _e4m3_values()
    cu_q, cu_k = _ragged([25], [25])
    kc = _fp8_keys_case(67, 25, 16)
    qc = _fp8_keys_case(68, 25, 2 * 16).reshape(25, 2, 16)
    sc = np.random.default_rng(69).integers(120, 134, 25).astype(np.uint8)
    w = np.random.default_rng(70).standard_normal((25, 2)).astype(np.float32)
    g = np.tril(np.random.default_rng(71).standard_normal((25, 25)))
    got = oracle.indexer_backward(cu_q, cu_k, qc, kc, w, g, k_scale=sc)
    kf = (vals[kc] * 2.0 ** (sc.astype(np.int64) - 127)[:, None]).astype(np.float32)
    want = oracle.indexer_backward(cu_q, cu_k, vals[qc].astype(np.float32), kf, w, g)
    for a_, b_ in zip(got, want):
        np.testing.assert_allclose(a_, b_, rtol=1e-13, atol=1e-300)


# ------------------------------------------------- sparse attention backward

def _torch_attn_grads(cu_q, cu_k, q, kv, idx, d_v, scale, dout):
    """Gradients of sum(dout * out) through torch's autograd, the sparse MQA
    attention built from torch ops in float64 (gather, softmax, matmul)."""
    pos, base = _positions(cu_q, cu_k)
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(kv, dtype=torch.float64, requires_grad=True)
    total = torch.zeros((), dtype=torch.float64)
    for i in range(len(pos)):
        sel = idx[i][idx[i] >= 0]
        if len(sel) == 0:
            continue
        c = kt[torch.from_numpy(base[i] + sel)]
        pr = torch.softmax(scale * qt[i] @ c.T, dim=-1)
        out = pr @ c[:, :d_v]
        total = total + (torch.from_numpy(dout[i]) * out).sum()
    total.backward()
    return qt.grad.numpy(), kt.grad.numpy()


def test_sparse_attention_backward_matches_torch_autograd():
    rng = np.random.default_rng(72)
    cu_q, cu_k = _ragged([40, 26, 9], [40, 3, 1])
    pos, _ = _positions(cu_q, cu_k)
    H, d_qk, d_v, k = 3, 24, 16, 10
    q = rng.standard_normal((len(pos), H, d_qk)).astype(np.float32)
    kv = rng.standard_normal((int(cu_k[-1]), d_qk)).astype(np.float32)
    idx = np.full((len(pos), k), -1, np.int32)
    for i in range(len(pos)):
        n = pos[i] + 1
        sel = np.sort(rng.choice(n, min(n, k), replace=False))
        idx[i, :len(sel)] = sel
    idx[5, :] = -1                                  # an empty selection: no gradient
    dout = rng.standard_normal((len(pos), H, d_v))
    dq, dkv = oracle.sparse_mla_backward(cu_q, cu_k, q, kv, idx, d_v, 0.3, dout)
    rq, rk = _torch_attn_grads(cu_q, cu_k, q, kv, idx, d_v, 0.3, dout)
    np.testing.assert_allclose(dq, rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dkv, rk, rtol=1e-10, atol=1e-12)
    assert np.all(dq[5] == 0.0)
    # rows nobody selected get no gradient
    chosen = np.zeros(len(kv), bool)
    for i in range(len(pos)):
        chosen[_positions(cu_q, cu_k)[1][i] + idx[i][idx[i] >= 0]] = True
    assert np.all(dkv[~chosen] == 0.0)


def test_sparse_attention_backward_closed_forms():
    """One selected entry: P = 1, so dq = 0 and that row's gradient is dout on
    the value columns only; a zero upstream gives zero gradients."""
    rng = np.random.default_rng(73)
    cu_q, cu_k = _ragged([5], [5])
    q = rng.standard_normal((5, 2, 6)).astype(np.float32)
    kv = rng.standard_normal((5, 6)).astype(np.float32)
    idx = np.array([[0, -1], [1, -1], [0, -1], [3, -1], [2, -1]], np.int32)
    dout = rng.standard_normal((5, 2, 4))
    dq, dkv = oracle.sparse_mla_backward(cu_q, cu_k, q, kv, idx, 4, 0.5, dout)
    assert np.max(np.abs(dq)) < 1e-15
    want = np.zeros((5, 6))
    for i in range(5):
        want[idx[i, 0], :4] += dout[i].sum(0)
    np.testing.assert_allclose(dkv, want, atol=1e-14)
    z = oracle.sparse_mla_backward(cu_q, cu_k, q, kv, idx, 4, 0.5, np.zeros_like(dout))
    assert np.all(z[0] == 0.0) and np.all(z[1] == 0.0)


# ---------------------------------------------------------------- end to end

def test_forward_composes_the_steps_and_is_causal():
    p = gen.make_problem("t", [96, 40], [96, 3], H_I=2, d_I=8, H=2, d_qk=16, d_v=8, k=16,
                         idx_dtype=torch.float32, dtype=torch.float32, seed=4)
    a = dict(q_idx=gen.storage_numpy(p.q_idx), k_idx=gen.storage_numpy(p.k_idx), w=gen.storage_numpy(p.w),
             q=gen.storage_numpy(p.q), kv=gen.storage_numpy(p.kv))
    out, lse, sc, idx = oracle.forward(p.cu_q_host, p.cu_k_host, a["q_idx"], a["k_idx"], a["w"], a["q"], a["kv"],
                                       p.k, p.d_v, p.scale)
    s_sep = oracle.indexer(p.cu_q_host, p.cu_k_host, a["q_idx"], a["k_idx"], a["w"], ld=sc.shape[1])
    i_sep = oracle.topk(p.cu_q_host, p.cu_k_host, s_sep.astype(np.float32), p.k)
    o_sep, l_sep = oracle.sparse_mla(p.cu_q_host, p.cu_k_host, a["q"], a["kv"], i_sep, p.d_v, p.scale)
    assert np.array_equal(idx, i_sep) and np.array_equal(out, o_sep) and np.array_equal(lse, l_sep)
    # perturb every token after position 50 of sequence 0: rows <= 50 unchanged
    kv2, kidx2 = a["kv"].copy(), a["k_idx"].copy()
    kv2[51:96] += 3.0
    kidx2[51:96] *= -2.0
    out2, lse2, _, idx2 = oracle.forward(p.cu_q_host, p.cu_k_host, a["q_idx"], kidx2, a["w"], a["q"], kv2,
                                         p.k, p.d_v, p.scale)
    assert np.array_equal(out2[:51], out[:51]) and np.array_equal(idx2[:51], idx[:51])
    assert np.array_equal(out2[96:], out[96:])   # the other sequence is independent
    assert not np.array_equal(out2[51:96], out[51:96])


def test_forward_rows_subset_matches_full():
    p = gen.make_problem("t", [70], [70], H_I=2, d_I=8, H=2, d_qk=16, d_v=8, k=16,
                         idx_dtype=torch.float32, dtype=torch.float32, seed=6)
    arr = [gen.storage_numpy(t) for t in (p.q_idx, p.k_idx, p.w, p.q, p.kv)]
    full = oracle.forward(p.cu_q_host, p.cu_k_host, *arr, p.k, p.d_v, p.scale)
    rows = np.array([0, 15, 16, 69], np.int32)
    sub = oracle.forward(p.cu_q_host, p.cu_k_host, arr[0][rows], arr[1], arr[2][rows], arr[3][rows], arr[4],
                         p.k, p.d_v, p.scale, rows=rows, ld=70)
    for a, b in zip(sub, full):
        assert np.array_equal(a, b[rows])
