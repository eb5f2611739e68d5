"""Tensor-level helpers over libdsa: allocate outputs and workspaces with torch
(device memory and streams only) and call the C entry points.  No arithmetic
of the method happens here."""
from __future__ import annotations

import torch

from . import libdsa as L


def _ws(nbytes: int, device):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def score_ld(max_ctx: int) -> int:
    return (int(max_ctx) + 63) // 64 * 64


def indexer_scores(p, act=L.DSA_ACT_RELU, ld=None, fill=float("nan")):
    """Scores [total_q, ld] fp32; entries beyond each row's causal bound keep `fill`."""
    ld = score_ld(p.max_ctx) if ld is None else ld
    scores = torch.full((p.total_q, ld), fill, dtype=torch.float32, device=p.q_idx.device)
    b = L.batch_of(p)
    n = L.dsa_indexer_workspace_size(b, p.q_idx, act)
    L.dsa_indexer_scores(b, p.q_idx, p.k_idx, p.w, scores, act=act, ws=_ws(n, scores.device) if n else None,
                         k_idx_scale=p.k_idx_scale)
    return scores


def topk(p, scores, k=None):
    k = p.k if k is None else k
    b = L.batch_of(p)
    idx = torch.empty((p.total_q, k), dtype=torch.int32, device=scores.device)
    n = L.dsa_topk_workspace_size(b, k)
    L.dsa_topk(b, scores, k, idx, ws=_ws(n, scores.device) if n else None)
    return idx


def sparse_mla_attn(p, idx, with_lse=True):
    b = L.batch_of(p)
    dev = p.q.device
    out = torch.empty((p.total_q, p.H, p.d_v), dtype=p.q.dtype, device=dev)
    lse = torch.empty((p.total_q, p.H), dtype=torch.float32, device=dev) if with_lse else None
    n = L.dsa_sparse_mla_attn_workspace_size(b, L._dtype_code(p.q), p.H, idx.shape[1], p.d_qk, p.d_v)
    L.dsa_sparse_mla_attn(b, p.q, p.kv, idx, p.d_v, p.scale, out, lse, ws=_ws(n, dev) if n else None)
    return out, lse


def dense_mla_attn(p, with_lse=True):
    """Dense causal MQA over every candidate [0, pos] (the masked mode)."""
    b = L.batch_of(p)
    dev = p.q.device
    out = torch.empty((p.total_q, p.H, p.d_v), dtype=p.q.dtype, device=dev)
    lse = torch.empty((p.total_q, p.H), dtype=torch.float32, device=dev) if with_lse else None
    n = L.dsa_dense_mla_attn_workspace_size(b, L._dtype_code(p.q), p.H, p.d_qk, p.d_v)
    L.dsa_dense_mla_attn(b, p.q, p.kv, p.d_v, p.scale, out, lse, ws=_ws(n, dev) if n else None)
    return out, lse


class Forward:
    """A prepared dsa_forward call: outputs and workspace allocated once, so
    that repeated calls (benchmarks) allocate nothing."""

    def __init__(self, p, act=L.DSA_ACT_RELU, q_block=None, with_idx=True, with_lse=True):
        dev = p.q.device
        self.p = p
        self.batch = L.batch_of(p)
        self.out = torch.empty((p.total_q, p.H, p.d_v), dtype=p.q.dtype, device=dev)
        self.lse = torch.empty((p.total_q, p.H), dtype=torch.float32, device=dev) if with_lse else None
        self.idx = torch.empty((p.total_q, p.k), dtype=torch.int32, device=dev) if with_idx else None
        qb = p.q_block if q_block is None else q_block
        self.params = L.forward_params(self.batch, p.q_idx, p.k_idx, p.w, p.q, p.kv, p.k, p.d_v, p.scale,
                                       self.out, self.lse, self.idx, act=act, q_block=qb,
                                       k_idx_scale=p.k_idx_scale)
        self.ws = _ws(L.dsa_forward_workspace_size(self.params), dev)

    def __call__(self, stream=None):
        L.dsa_forward(self.params, self.ws, stream=stream)
        return self.out, self.lse, self.idx


def cache_append(k_new=None, k_cache=None, k_scale=None, kv_new=None, kv_cache=None, dst_rows=None):
    """Write new tokens into the caches (indexer keys quantised to E4M3, optional
    per-token E8M0 scales; latent rows copied); see dsa_cache_append."""
    L.dsa_cache_append(k_new=k_new, k_cache=k_cache, k_scale=k_scale, kv_new=kv_new, kv_cache=kv_cache,
                       dst_rows=dst_rows)


def forward(p, act=L.DSA_ACT_RELU, q_block=None):
    f = Forward(p, act=act, q_block=q_block)
    return f()
