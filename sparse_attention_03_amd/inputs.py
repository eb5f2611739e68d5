"""Seeded synthetic inputs for the DSA hot path.

This module only draws random tensors and stores them in the element formats
the library consumes; it holds none of the method's arithmetic.  The same bytes
feed the library and the CPU oracle: a caller generates once, on any device,
and copies to the host for the oracle.

Distributions follow the workload descriptions of the five standard
configurations (named after what they are):

* ``tiny_fp32``      -- 1 sequence, L=256, fp32 throughout; H_I=4, d_I=32, k=32,
  8 query heads over one latent (d_qk=80, d_v=64); q, k ~ N(0,1)/sqrt(d),
  w ~ U(0,1).
* ``prefill_8k``     -- 1 sequence, L=8192; H_I=64, d_I=128 e4m3 from
  N(0,1)/sqrt(128); w ~ U(0,1)/8; k=2048; 128 heads, bf16 q [L,128,576] and
  latent [L,576] from N(0,1); d_v=512; scale 1/sqrt(192).
* ``decode_64x32k``  -- 64 sequences, one new query each, 32768-token caches.
* ``prefill_128k``   -- 1 sequence, L=131072, processed in 4096-query chunks.
* ``decode_mixed``   -- 32 sequences with lengths U{4096..131072} plus 8 of
  length 1024 (fewer candidates than k), one query each.

Random numbers come from torch's seeded generator on the target device
(Philox on the GPU, mt19937 on the CPU).  FP8 values are produced by torch's
float32 -> float8_e4m3fn cast (round to nearest even; every drawn value is far
inside the +-448 range), bf16 values by torch's float32 -> bfloat16 cast.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3 = torch.float8_e4m3fn


@dataclass
class DSAInputs:
    """One synthetic problem.  Tensors live on ``device``; cu_* also on host."""
    name: str
    cu_q: torch.Tensor            # int32 [B+1] on device
    cu_k: torch.Tensor            # int32 [B+1] on device
    cu_q_host: np.ndarray         # int32 [B+1]
    cu_k_host: np.ndarray         # int32 [B+1]
    q_idx: torch.Tensor           # [T, H_I, d_I] e4m3 or fp32
    k_idx: torch.Tensor           # [total_k, d_I] same dtype
    w: torch.Tensor               # [T, H_I] fp32
    q: torch.Tensor               # [T, H, d_qk] bf16 or fp32
    kv: torch.Tensor              # [total_k, d_qk] same dtype
    k: int
    d_v: int
    scale: float
    q_block: int = 0
    meta: dict = field(default_factory=dict)
    k_idx_scale: torch.Tensor | None = None   # uint8 [total_k] E8M0 per-token key scales, or None

    @property
    def total_q(self) -> int:
        return int(self.cu_q_host[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_k_host[-1])

    @property
    def max_ctx(self) -> int:
        return int(np.max(np.diff(self.cu_k_host)))

    @property
    def num_seqs(self) -> int:
        return len(self.cu_q_host) - 1

    @property
    def H_I(self) -> int:
        return self.q_idx.shape[1]

    @property
    def d_I(self) -> int:
        return self.q_idx.shape[2]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def d_qk(self) -> int:
        return self.q.shape[2]

    def positions(self) -> np.ndarray:
        """Absolute position of every query row (host)."""
        pos = np.empty(self.total_q, dtype=np.int64)
        for b in range(self.num_seqs):
            q0, q1 = self.cu_q_host[b], self.cu_q_host[b + 1]
            ctx = self.cu_k_host[b + 1] - self.cu_k_host[b]
            pos[q0:q1] = ctx - (q1 - q0) + np.arange(q1 - q0)
        return pos


def storage_numpy(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as numpy: fp32 -> float32, bf16 -> uint16 bits,
    e4m3 -> uint8 codes, integers as they are."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == E4M3:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, std, out_dtype, chunk_elems=1 << 28, keep=None):
    """N(0, std^2) drawn in float32 and stored as out_dtype, in chunks to bound
    the float32 temporary.  `keep`: a list that receives the float32 draws
    before the storage cast (the same random stream either way)."""
    shape = tuple(int(s) for s in shape)
    n = math.prod(shape)
    if out_dtype == torch.bfloat16 and std == 1.0 and keep is None:
        return torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
    out = torch.empty(n, dtype=out_dtype, device=device)
    full = torch.empty(n, dtype=torch.float32, device=device) if keep is not None else None
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[s:e] = x.to(out_dtype)
        if full is not None:
            full[s:e] = x
    if keep is not None:
        keep.append(full.view(shape))
    return out.view(shape)


def _integer_values(shape, g, device, lo, hi, out_dtype):
    x = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return x.to(torch.float32).to(out_dtype)


def make_problem(name, seq_ctx, seq_q, *, H_I=64, d_I=128, H=128, d_qk=576, d_v=512, k=2048,
                 idx_dtype=E4M3, dtype=torch.bfloat16, w_scale=0.125, qk_std=None, kv_std=1.0,
                 q_std=None, scale=None, device="cpu", seed=0, integer=False, q_block=0,
                 keep_unquantised=False):
    """General ragged problem: sequence b has seq_ctx[b] cached tokens (the
    query rows included) and its last seq_q[b] tokens are the queries.
    keep_unquantised: also keep the float32 draws of q_idx and k_idx (before
    their storage cast) in meta["q_idx_f32"] / meta["k_idx_f32"]."""
    seq_ctx = [int(c) for c in seq_ctx]
    seq_q = [int(x) for x in seq_q]
    assert len(seq_ctx) == len(seq_q) and all(0 < qq <= c for qq, c in zip(seq_q, seq_ctx))
    cu_q = np.zeros(len(seq_q) + 1, dtype=np.int32)
    cu_k = np.zeros(len(seq_ctx) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(seq_q)
    cu_k[1:] = np.cumsum(seq_ctx)
    T, K = int(cu_q[-1]), int(cu_k[-1])
    g = _gen(device, seed)
    if qk_std is None:
        qk_std = 1.0 / math.sqrt(d_I)
    if q_std is None:
        q_std = 1.0
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    if integer:
        # integer-valued: every fp8/fp32 product and partial sum is exact
        q_idx = _integer_values((T, H_I, d_I), g, device, -4, 4, idx_dtype)
        k_idx = _integer_values((K, d_I), g, device, -4, 4, idx_dtype)
        w = torch.randint(0, 9, (T, H_I), generator=g, device=device, dtype=torch.int32).to(torch.float32) * 0.25
    else:
        kq, kk = ([], []) if keep_unquantised else (None, None)
        q_idx = _normal((T, H_I, d_I), g, device, qk_std, idx_dtype, keep=kq)
        k_idx = _normal((K, d_I), g, device, qk_std, idx_dtype, keep=kk)
        w = torch.rand((T, H_I), generator=g, device=device, dtype=torch.float32) * w_scale
    q = _normal((T, H, d_qk), g, device, q_std, dtype)
    kv = _normal((K, d_qk), g, device, kv_std, dtype)
    meta = dict(seed=seed, integer=integer)
    if keep_unquantised and not integer:
        meta["q_idx_f32"], meta["k_idx_f32"] = kq[0], kk[0]
    return DSAInputs(name=name,
                     cu_q=torch.from_numpy(cu_q).to(device), cu_k=torch.from_numpy(cu_k).to(device),
                     cu_q_host=cu_q, cu_k_host=cu_k, q_idx=q_idx, k_idx=k_idx, w=w, q=q, kv=kv,
                     k=k, d_v=d_v, scale=float(scale), q_block=q_block, meta=meta)


def mixed_decode_lengths(seed=0, n_long=32, n_short=8, lo=4096, hi=131072, short=1024):
    """Context lengths of the mixed decode batch: n_long drawn U{lo..hi} from the
    seed (host generator, so every device sees the same lengths), then n_short
    sequences of length `short`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    longs = rng.integers(lo, hi + 1, size=n_long)
    return [int(x) for x in longs] + [short] * n_short


CONFIGS = ("tiny_fp32", "prefill_8k", "decode_64x32k", "prefill_128k", "decode_mixed")


def make_config(name, device="cpu", seed=0, **over):
    """The five standard workloads (see module docstring)."""
    if name == "tiny_fp32":
        kw = dict(H_I=4, d_I=32, H=8, d_qk=80, d_v=64, k=32, idx_dtype=torch.float32,
                  dtype=torch.float32, w_scale=1.0, qk_std=1 / math.sqrt(32), kv_std=1 / math.sqrt(80),
                  q_std=1 / math.sqrt(80), scale=1 / math.sqrt(80))
        kw.update(over)
        return make_problem(name, [256], [256], device=device, seed=seed, **kw)
    if name == "prefill_8k":
        return make_problem(name, [8192], [8192], device=device, seed=seed, **over)
    if name == "decode_64x32k":
        return make_problem(name, [32768] * 64, [1] * 64, device=device, seed=seed, **over)
    if name == "prefill_128k":
        over.setdefault("q_block", 4096)
        return make_problem(name, [131072], [131072], device=device, seed=seed, **over)
    if name == "decode_mixed":
        lens = mixed_decode_lengths(seed)
        return make_problem(name, lens, [1] * len(lens), device=device, seed=seed, **over)
    raise KeyError(name)
