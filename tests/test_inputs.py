"""Seeded input generator: determinism, shapes, formats, configuration recipes."""
import math

import numpy as np
import torch

from sparse_attention_03_amd import inputs as gen


def test_same_seed_same_bytes_and_different_seed_differs():
    a = gen.make_problem("x", [64, 33], [64, 1], H_I=16, d_I=128, H=32, seed=5)
    b = gen.make_problem("x", [64, 33], [64, 1], H_I=16, d_I=128, H=32, seed=5)
    c = gen.make_problem("x", [64, 33], [64, 1], H_I=16, d_I=128, H=32, seed=6)
    for n in ("q_idx", "k_idx", "w", "q", "kv"):
        assert np.array_equal(gen.storage_numpy(getattr(a, n)), gen.storage_numpy(getattr(b, n)))
        assert not np.array_equal(gen.storage_numpy(getattr(a, n)), gen.storage_numpy(getattr(c, n)))


def test_ragged_layout_and_positions():
    p = gen.make_problem("x", [10, 7, 5], [10, 2, 1], H_I=16, H=32, seed=0)
    assert list(p.cu_q_host) == [0, 10, 12, 13] and list(p.cu_k_host) == [0, 10, 17, 22]
    assert list(p.positions()) == list(range(10)) + [5, 6, 4]
    assert p.q_idx.dtype == torch.float8_e4m3fn and p.q.dtype == torch.bfloat16
    assert p.q_idx.shape == (13, 16, 128) and p.k_idx.shape == (22, 128) and p.kv.shape == (22, 576)


def test_distributions_follow_the_recipe():
    p = gen.make_problem("x", [4096], [4096], H_I=16, H=8, seed=1)
    qi = p.q_idx.float()
    assert abs(qi.std().item() - 1 / math.sqrt(128)) < 0.01
    assert 0.0 <= p.w.min().item() and p.w.max().item() <= 0.125
    assert abs(p.kv.float().std().item() - 1.0) < 0.02


def test_integer_inputs_are_small_integers():
    p = gen.make_problem("x", [50], [50], H_I=16, H=8, integer=True, seed=2)
    v = p.q_idx.float()
    assert torch.equal(v, v.round()) and v.abs().max() <= 4
    assert torch.equal(p.w * 4, (p.w * 4).round())


def test_mixed_decode_lengths():
    lens = gen.mixed_decode_lengths(0)
    assert len(lens) == 40 and lens[32:] == [1024] * 8
    assert all(4096 <= x <= 131072 for x in lens[:32])
    assert lens == gen.mixed_decode_lengths(0)


def test_tiny_config():
    p = gen.make_config("tiny_fp32")
    assert p.q_idx.dtype == torch.float32 and p.q.shape == (256, 8, 80) and p.k == 32 and p.d_v == 64
    assert abs(p.scale - 1 / math.sqrt(80)) < 1e-12


def test_unquantised_draws_are_the_same_stream():
    """keep_unquantised changes nothing in the stored inputs, and the kept
    float32 draws cast to E4M3 are exactly the stored codes."""
    a = gen.make_problem("x", [70, 20], [70, 1], H_I=16, H=8, seed=4)
    b = gen.make_problem("x", [70, 20], [70, 1], H_I=16, H=8, seed=4, keep_unquantised=True)
    for n in ("q_idx", "k_idx", "w", "q", "kv"):
        assert np.array_equal(gen.storage_numpy(getattr(a, n)), gen.storage_numpy(getattr(b, n)))
    assert "q_idx_f32" not in a.meta
    for n in ("q_idx", "k_idx"):
        f = b.meta[n + "_f32"]
        assert f.dtype == torch.float32 and f.shape == getattr(b, n).shape
        assert np.array_equal(gen.storage_numpy(f.to(gen.E4M3)), gen.storage_numpy(getattr(b, n)))
