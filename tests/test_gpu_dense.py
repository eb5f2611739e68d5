"""Parity of dsa_dense_mla_attn (HIP, the masked mode of short prefill)
against the CPU oracle, and its bit-identity with the sparse kernel over
every candidate."""
import numpy as np
import pytest
import torch

import oracle
from dsa_check import TOL_ATTN_BF16, TOL_ATTN_F32, announce, host, row_norm_err
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_03_amd import dsa as d
    return d


def _oracle_dense(p, rows):
    q = host(p.q)[rows]
    return oracle.dense_mla(p.cu_q_host, p.cu_k_host, q, host(p.kv), p.d_v, p.scale, rows=rows)


def _check(p, out, lse, rows, tol):
    ref_o, ref_l = _oracle_dense(p, rows)
    got = out.float().cpu().numpy()[rows]
    err = row_norm_err(got, ref_o)
    lerr = float(np.max(np.abs(lse.cpu().numpy()[rows] - ref_l)))
    print(f"row-normalised error {err:.3e}, lse abs error {lerr:.3e}")
    assert err <= tol
    assert lerr <= (1e-2 if tol >= 1e-3 else 1e-4)


@pytest.mark.parametrize("H", [16, 32, 64, 96, 128])
def test_dense_bf16_prefill_rows(dsa, H):
    """A prefill sequence of 700 rows (several tiles, a ragged last tile) and a
    one-token sequence; sampled rows against the oracle."""
    announce("dense attention bf16 prefill", H)
    p = gen.make_problem("dense", [700, 1], [700, 1], H_I=16, H=H, k=2048, device=DEV, seed=H)
    out, lse = dsa.dense_mla_attn(p)
    rows = [0, 1, 31, 32, 33, 95, 300, 511, 698, 699, 700]
    _check(p, out, lse, rows, TOL_ATTN_BF16)


def test_dense_bf16_decode_rows_use_key_splits(dsa):
    """Few long rows: the keys are split over workgroups and merged."""
    announce("dense attention bf16 decode split")
    p = gen.make_problem("dense", [9000, 4097, 64, 2500], [1, 2, 1, 1], H_I=16, H=128, k=2048, device=DEV, seed=3)
    out, lse = dsa.dense_mla_attn(p)
    _check(p, out, lse, list(range(p.total_q)), TOL_ATTN_BF16)


@pytest.mark.parametrize("ctx", [4100, 9000, 70000])
def test_dense_bf16_one_row_many_key_splits(dsa, ctx):
    """One long row: it is split over keys into 128 or 256 parts (more than a
    wave's worth), all of which the merge must weigh."""
    announce("dense attention bf16 one row, many splits", ctx)
    p = gen.make_problem("dense", [ctx], [1], H_I=16, H=128, k=2048, device=DEV, seed=ctx)
    out, lse = dsa.dense_mla_attn(p)
    _check(p, out, lse, [0], TOL_ATTN_BF16)


@pytest.mark.parametrize("d_qk,d_v", [(128, 64), (576, 128)])
def test_dense_bf16_narrow_widths(dsa, d_qk, d_v):
    """The masked mode with BF16 widths other than 576 / 512 (widened copies)."""
    announce("dense attention bf16 widths", d_qk, d_v)
    p = gen.make_problem("dense", [700, 1], [700, 1], H_I=16, H=32, d_qk=d_qk, d_v=d_v, k=2048, device=DEV, seed=3)
    out, lse = dsa.dense_mla_attn(p)
    _check(p, out, lse, [0, 1, 31, 32, 300, 699, 700], TOL_ATTN_BF16)


def test_dense_equals_sparse_over_every_candidate(dsa):
    """With as many rows as compute units neither call splits rows, and the
    dense kernel walks the same tiles in the same order as the sparse kernel
    given idx = 0 .. pos: the results are bit-identical."""
    announce("dense vs sparse bit identity")
    p = gen.make_problem("dense", [1500, 900], [400, 300], H_I=16, H=128, k=2048, device=DEV, seed=5)
    pos = p.positions()
    idx = -np.ones((p.total_q, 2048), np.int32)
    for i, ps in enumerate(pos):
        idx[i, :ps + 1] = np.arange(ps + 1)
    out_d, lse_d = dsa.dense_mla_attn(p)
    out_s, lse_s = dsa.sparse_mla_attn(p, torch.from_numpy(idx).to(DEV))
    assert torch.equal(out_d, out_s)
    assert torch.equal(lse_d, lse_s)


def test_dense_f32_tiny_config(dsa):
    announce("dense attention f32 tiny")
    p = gen.make_config("tiny_fp32", device=DEV)
    out, lse = dsa.dense_mla_attn(p)
    _check(p, out, lse, list(range(p.total_q)), TOL_ATTN_F32)
