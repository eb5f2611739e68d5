"""dsa_cache_append (HIP) against the CPU oracle: E4M3FN codes and E8M0 scales
bit for bit, latent rows copied, destinations honoured; and the indexer /
forward with per-token key scales against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import MIN_RECALL, TOL_ATTN_BF16, TOL_SCORES_FP8, announce, causal_mask, host, oracle_attention_on, recall, \
    row_norm_err, rows_of
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_03_amd import dsa as d
    return d


def _e4m3_values():
    return np.array([oracle.e4m3_value(c) for c in range(256)])


def _append_keys(dsa, k_new, scaled, dst=None, cache_rows=None, fill=0xAB):
    n, d = k_new.shape
    rows = n if cache_rows is None else cache_rows
    kc = torch.full((rows, d), fill, dtype=torch.uint8, device=DEV)
    ks = torch.full((rows,), fill, dtype=torch.uint8, device=DEV) if scaled else None
    dsa.cache_append(k_new=k_new, k_cache=kc, k_scale=ks, dst_rows=dst)
    torch.cuda.synchronize()
    return kc.cpu().numpy(), (ks.cpu().numpy() if scaled else None)


def _special_f32():
    """Every E4M3 value, the midpoints between neighbours and the floats just
    beside them, saturation, infinities, NaN, signed zeros, fp32 denormals."""
    vals = _e4m3_values()
    pos = np.array([vals[c] for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    xs = [pos.astype(np.float32), m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
          np.array([448, 449, 463.9, 464, 464.1, 479, 480, 500, 1e30, 3e38, np.inf, np.nan, 0.0, 1e-40, 1e-45,
                    2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -11, 2.0 ** -12], np.float32)]
    x = np.concatenate(xs).astype(np.float32)
    return np.concatenate([x, -x])   # the negated half holds -0.0 and -NaN too


@pytest.mark.parametrize("d_I", [64, 128, 256, 512])
def test_fp32_special_values_unscaled(dsa, d_I):
    announce("cache append fp32 specials", d_I)
    x = _special_f32()
    rng = np.random.default_rng(41)
    extra = (rng.standard_normal(4096) * np.exp2(rng.uniform(-14, 10, 4096))).astype(np.float32)
    x = np.concatenate([x, extra])
    n = (len(x) + d_I - 1) // d_I
    x = np.concatenate([x, np.zeros(n * d_I - len(x), np.float32)]).reshape(n, d_I)
    got, _ = _append_keys(dsa, torch.from_numpy(x).to(DEV), scaled=False)
    assert np.array_equal(got, oracle.quantize_keys(x))


def test_bf16_every_bit_pattern(dsa):
    announce("cache append bf16 every pattern")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    k_new = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    got, _ = _append_keys(dsa, k_new, scaled=False)
    assert np.array_equal(got, oracle.quantize_keys(bits))


def _scaled_rows(seed, n, d):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)) * np.exp2(rng.uniform(-40, 40, (n, 1)))
    x = x.astype(np.float32)
    x[0] = 0.0                                   # e = 0
    x[1] = 0.5
    x[1, 3] = 448.0 * 2.0 ** 5                   # amax exactly 448 * 2^5: e = 5
    x[2] = 0.5
    x[2, 3] = np.nextafter(np.float32(448.0 * 2.0 ** 5), np.float32(1e30))  # e = 6
    x[3, 7] = np.inf                             # e = 127
    x[4, 9] = np.nan                             # ignored by the maximum, coded 0x7F
    x[5] = 1e-44                                 # fp32 denormals only: e clamps at -127
    x[6] = -3e38                                 # largest magnitudes: e = 120
    x[7, ::2] = -0.0
    return x


@pytest.mark.parametrize("d_I", [64, 128, 512])
def test_fp32_per_token_scale(dsa, d_I):
    announce("cache append fp32 scaled", d_I)
    x = _scaled_rows(42, 300, d_I)
    got, sc = _append_keys(dsa, torch.from_numpy(x).to(DEV), scaled=True)
    want, want_sc = oracle.quantize_keys(x, scaled=True)
    assert np.array_equal(sc, want_sc)
    assert list(sc[:7].astype(int) - 127) == [0, 5, 6, 127, int(want_sc[4]) - 127, -127, 120]
    assert np.array_equal(got, want)


def test_bf16_per_token_scale(dsa):
    announce("cache append bf16 scaled")
    x = torch.from_numpy(_scaled_rows(43, 257, 128)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    got, sc = _append_keys(dsa, x.to(DEV), scaled=True)
    want, want_sc = oracle.quantize_keys(bits, scaled=True)
    assert np.array_equal(sc, want_sc)
    assert np.array_equal(got, want)


def test_destination_rows_and_latent_copy(dsa):
    """Tokens go to dst_rows[t]; rows outside [0, cache_rows) are dropped; rows
    nobody writes keep their old bytes; the latent part is a byte copy."""
    announce("cache append destinations + latent")
    n, rows = 777, 1500
    rng = np.random.default_rng(44)
    dst = rng.permutation(rows)[:n].astype(np.int32)
    dst[5], dst[6], dst[700] = -1, rows, 2 ** 30
    x = _scaled_rows(45, n, 128)
    for kv_dtype in (torch.bfloat16, torch.float32):
        kv_new = torch.randn((n, 576), dtype=torch.float32, device=DEV).to(kv_dtype)
        kv_cache = torch.full((rows, 576), 7.0, dtype=kv_dtype, device=DEV)
        kc = torch.full((rows, 128), 0xAB, dtype=torch.uint8, device=DEV)
        ks = torch.full((rows,), 0xCD, dtype=torch.uint8, device=DEV)
        d_dst = torch.from_numpy(dst).to(DEV)
        dsa.cache_append(k_new=torch.from_numpy(x).to(DEV), k_cache=kc, k_scale=ks, kv_new=kv_new,
                         kv_cache=kv_cache, dst_rows=d_dst)
        torch.cuda.synchronize()
        codes, sc = oracle.quantize_keys(x, scaled=True)
        want_kc = np.full((rows, 128), 0xAB, np.uint8)
        want_ks = np.full(rows, 0xCD, np.uint8)
        want_kv = torch.full((rows, 576), 7.0, dtype=kv_dtype)
        ok = (dst >= 0) & (dst < rows)
        want_kc[dst[ok]] = codes[ok]
        want_ks[dst[ok]] = sc[ok]
        want_kv[torch.from_numpy(dst[ok]).long()] = kv_new.cpu()[torch.from_numpy(np.nonzero(ok)[0])]
        assert np.array_equal(kc.cpu().numpy(), want_kc)
        assert np.array_equal(ks.cpu().numpy(), want_ks)
        assert torch.equal(kv_cache.cpu().view(torch.uint8), want_kv.view(torch.uint8))
    # latent only, identity destinations, a ragged tail of 16-byte chunks
    kv_new = torch.randn((1001, 576), dtype=torch.bfloat16, device=DEV)
    kv_cache = torch.zeros_like(kv_new)
    dsa.cache_append(kv_new=kv_new, kv_cache=kv_cache)
    assert torch.equal(kv_cache, kv_new)
    # keys only, unscaled
    got, _ = _append_keys(dsa, torch.from_numpy(x).to(DEV), scaled=False, dst=torch.from_numpy(dst).to(DEV),
                          cache_rows=rows)
    want_kc = np.full((rows, 128), 0xAB, np.uint8)
    want_kc[dst[ok]] = oracle.quantize_keys(x)[ok]
    assert np.array_equal(got, want_kc)


# ------------------------------------------------- indexer with key scales

def _with_scales(p, seed, spread=3):
    rng = np.random.default_rng(seed)
    sc = rng.integers(127 - spread, 127 + spread + 1, p.total_k).astype(np.uint8)
    p.k_idx_scale = torch.from_numpy(sc).to(DEV)
    return p


def _oracle_scores(p, act=0, ld=None):
    q_idx, w, _ = rows_of(p, None)
    return oracle.indexer(p.cu_q_host, p.cu_k_host, q_idx, host(p.k_idx), w, act=act, ld=ld,
                          k_scale=host(p.k_idx_scale))


@pytest.mark.parametrize("shape", ["prefill", "decode"])
@pytest.mark.parametrize("H_I,d_I", [(16, 128), (64, 128), (20, 64)])
def test_scaled_keys_integer_inputs_bit_exact(dsa, shape, H_I, d_I):
    """Integer-valued codes and power-of-two scales: every product and partial
    sum is exact, so the scores equal the oracle's bit for bit (workgroups of
    one sequence, workgroups spanning two, and the decode streaming kernel;
    d_I = 64 keys are widened with their scales unchanged)."""
    announce("indexer scaled keys integer", shape, H_I, d_I)
    if shape == "prefill":
        p = gen.make_problem("s", [300, 77, 1000, 129], [300, 5, 3, 64], H_I=H_I, d_I=d_I, H=32, k=64, integer=True,
                             device=DEV, seed=46)
    else:
        p = gen.make_problem("s", [2000, 3000, 700, 5000], [1, 1, 2, 1], H_I=H_I, d_I=d_I, H=32, k=64, integer=True,
                             device=DEV, seed=47)
    _with_scales(p, 48)
    got = dsa.indexer_scores(p).cpu().numpy()
    ld = got.shape[1]
    ref = _oracle_scores(p, ld=ld)
    mask = causal_mask(p, None, ld)
    assert np.array_equal(got[mask], ref[mask].astype(np.float32))


@pytest.mark.parametrize("act", [0, 1])
def test_scaled_keys_from_fp32_quantisation(dsa, act):
    """fp32 keys over a wide range of magnitudes, quantised with per-token
    scales by dsa_cache_append, scored with those scales: within the FP8 bar of
    the oracle on the same bytes, and much closer to the fp32 keys' scores than
    the same keys quantised without scales."""
    announce("indexer scaled keys from fp32", act)
    p = gen.make_problem("s", [1500, 900], [1500, 1], H_I=64, H=32, k=64, device=DEV, seed=49)
    rng = np.random.default_rng(50)
    k32 = (rng.standard_normal((p.total_k, 128)) / np.sqrt(128) * np.exp2(rng.uniform(-12, 12, (p.total_k, 1))))
    k32 = k32.astype(np.float32)
    kc = torch.empty((p.total_k, 128), dtype=torch.uint8, device=DEV)
    ks = torch.empty((p.total_k,), dtype=torch.uint8, device=DEV)
    dsa.cache_append(k_new=torch.from_numpy(k32).to(DEV), k_cache=kc, k_scale=ks)
    p.k_idx = kc.view(gen.E4M3)
    p.k_idx_scale = ks
    got = dsa.indexer_scores(p, act=act).cpu().numpy()
    ld = got.shape[1]
    ref = _oracle_scores(p, act=act, ld=ld)
    mask = causal_mask(p, None, ld)
    err = row_norm_err(got, ref, mask)
    print("row-normalised error vs oracle on the same bytes", err)
    # fp32 rounding only (same bytes); GELU's near-linear part lets the head
    # sum cancel in rows of few small scores, so the check is 1e-3, far inside
    # the FP8 bar
    assert err <= min(TOL_SCORES_FP8, 1e-3)
    # against the selection made from the unquantised keys (queries as their
    # E4M3 values): the per-token scale keeps small and large keys inside
    # E4M3's range, unscaled codes flush the small ones and saturate the large
    q_idx, w, _ = rows_of(p, None)
    q32 = _e4m3_values()[q_idx].astype(np.float32)
    exact = oracle.indexer(p.cu_q_host, p.cu_k_host, q32, k32, w, act=act, ld=ld)
    unscaled = oracle.indexer(p.cu_q_host, p.cu_k_host, q_idx, oracle.quantize_keys(k32), w, act=act, ld=ld)

    def sel(sc):
        return oracle.topk(p.cu_q_host, p.cu_k_host, np.where(mask, sc, 0.0).astype(np.float32), p.k)

    n = p.positions() + 1
    ref_sel = sel(exact)
    r_sc, r_un = recall(sel(got), ref_sel, n)[0], recall(sel(unscaled), ref_sel, n)[0]
    print(f"top-{p.k} recall against fp32 keys: scaled {r_sc:.4f}, unscaled codes {r_un:.4f}")
    assert r_sc > r_un


def test_forward_decode_append_with_scaled_keys(dsa):
    """A decode step: the new token of every sequence is appended (key quantised
    with its scale, latent row copied) at its cache row, then dsa_forward runs
    on the scaled cache; selection and attention agree with the oracle."""
    announce("forward decode after append")
    ctx = [3000, 2500, 4097, 1200, 2048, 3333]
    p = gen.make_problem("dec", ctx, [1] * len(ctx), H_I=64, H=64, k=512, device=DEV, seed=51)
    g = torch.Generator(device=DEV)
    g.manual_seed(52)
    k32 = torch.randn((p.total_k, 128), generator=g, device=DEV) / 11.3
    k32 *= torch.exp2(torch.randint(-6, 7, (p.total_k, 1), generator=g, device=DEV).float())
    kc = torch.empty((p.total_k, 128), dtype=torch.uint8, device=DEV)
    ks = torch.empty((p.total_k,), dtype=torch.uint8, device=DEV)
    last = torch.from_numpy(p.cu_k_host[1:] - 1).to(DEV).int()
    # the cache before the step (every row; the new rows are overwritten next)
    dsa.cache_append(k_new=k32, k_cache=kc, k_scale=ks)
    kv_cache = p.kv.clone()
    kv_cache[last.long()] = 0
    new_kv = p.kv[last.long()].contiguous()
    dsa.cache_append(k_new=k32[last.long()].contiguous(), k_cache=kc, k_scale=ks, kv_new=new_kv,
                     kv_cache=kv_cache, dst_rows=last)
    assert torch.equal(kv_cache, p.kv)
    p.k_idx = kc.view(gen.E4M3)
    p.k_idx_scale = ks
    out, _, idx = dsa.forward(p)
    rows = np.arange(p.total_q, dtype=np.int32)
    q_idx, w, q = rows_of(p, None)
    ref_out, _, _, ref_idx = oracle.forward(p.cu_q_host, p.cu_k_host, q_idx, host(p.k_idx), w, q, host(p.kv), p.k,
                                            p.d_v, p.scale, k_scale=host(p.k_idx_scale))
    g_idx = idx.cpu().numpy()
    rec, rec_min = recall(g_idx, ref_idx, p.positions()[rows] + 1)
    print(f"recall mean {rec:.5f} min {rec_min:.5f}")
    assert rec >= MIN_RECALL
    o_on, _ = oracle_attention_on(p, g_idx)
    assert row_norm_err(out.float().cpu().numpy(), o_on) <= TOL_ATTN_BF16
