"""ctypes binding of libdsa (include/libdsa.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors must be
contiguous CUDA (HIP) tensors; the calls are enqueued on torch's current
stream and return immediately.  Every step of the computation runs in the HIP
kernels of libdsa.so: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LIBDSA_PATH: another build of the library (e.g. the sanitized host build)
LIB_PATH = os.environ.get("LIBDSA_PATH") or os.path.join(_HERE, "lib", "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_ACT_RELU, DSA_ACT_GELU = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "or python sparse_attention_03_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

_p, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class DsaBatch(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("cu_q", _p), ("cu_k", _p),
                ("total_q", _i32), ("total_k", _i32), ("max_ctx", _i32)]


class DsaForwardParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.POINTER(DsaBatch)),
                ("q_idx", _p), ("k_idx", _p), ("idx_dtype", ctypes.c_int), ("k_idx_scale", _p), ("w", _p),
                ("H_I", _i32), ("d_I", _i32), ("act", ctypes.c_int),
                ("q", _p), ("kv", _p), ("dtype", ctypes.c_int),
                ("H", _i32), ("d_qk", _i32), ("d_v", _i32), ("softmax_scale", _f32),
                ("k", _i32), ("q_block", _i32),
                ("out", _p), ("lse", _p), ("out_idx", _p)]


_BP = ctypes.POINTER(DsaBatch)
_FP = ctypes.POINTER(DsaForwardParams)
_SIGS = {
    "dsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_version": ([], ctypes.c_char_p),
    "dsa_indexer_workspace_size": ([_BP, ctypes.c_int, _i32, _i32, ctypes.c_int, ctypes.POINTER(_sz)], ctypes.c_int),
    "dsa_indexer_scores": ([_BP, _p, _p, ctypes.c_int, _p, _p, _i32, _i32, ctypes.c_int, _p, _i64, _p, _sz, _p],
                           ctypes.c_int),
    "dsa_topk_workspace_size": ([_BP, _i32, ctypes.POINTER(_sz)], ctypes.c_int),
    "dsa_topk": ([_BP, _p, _i64, _i32, _p, _p, _sz, _p], ctypes.c_int),
    "dsa_sparse_mla_attn_workspace_size": ([_BP, ctypes.c_int, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)],
                                           ctypes.c_int),
    "dsa_sparse_mla_attn": ([_BP, _p, _p, ctypes.c_int, _p, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _sz, _p],
                            ctypes.c_int),
    "dsa_dense_mla_attn_workspace_size": ([_BP, ctypes.c_int, _i32, _i32, _i32, ctypes.POINTER(_sz)], ctypes.c_int),
    "dsa_dense_mla_attn": ([_BP, _p, _p, ctypes.c_int, _i32, _i32, _i32, _f32, _p, _p, _p, _sz, _p], ctypes.c_int),
    "dsa_sparse_mla_backward_workspace_size": ([_BP, _i32, _i32, ctypes.POINTER(_sz)], ctypes.c_int),
    "dsa_sparse_mla_backward": ([_BP, _p, _p, ctypes.c_int, _p, _i32, _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p,
                                 _sz, _p], ctypes.c_int),
    "dsa_attn_target": ([_BP, _p, _p, ctypes.c_int, _p, _i32, _i32, _i32, _f32, _p, _p, _i64, _p], ctypes.c_int),
    "dsa_indexer_kl": ([_BP, _p, _i64, _p, _i32, _p, _i64, _p, _p, _p], ctypes.c_int),
    "dsa_indexer_backward": ([_BP, _p, _p, ctypes.c_int, _p, _p, _i32, _i32, ctypes.c_int, _p, _i32, _p, _i64,
                              _p, _p, _p, _p], ctypes.c_int),
    "dsa_cache_append": ([_i64, _p, _i64, _p, ctypes.c_int, _i32, _p, _p, _p, ctypes.c_int, _i32, _p, _p],
                         ctypes.c_int),
    "dsa_forward_workspace_size": ([_FP, ctypes.POINTER(_sz)], ctypes.c_int),
    "dsa_forward": ([_FP, _p, _sz, _p], ctypes.c_int),
    "dsa_forward_noalloc": ([_FP, _p], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class DsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = _lib.dsa_status_string(status).decode()
        super().__init__(f"{what}: {name}: {_lib.dsa_last_error().decode()}")


def _check(status: int, what: str):
    if status != DSA_OK:
        raise DsaError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_batch(cu_q: torch.Tensor, cu_k: torch.Tensor, total_q: int, total_k: int, max_ctx: int) -> DsaBatch:
    """Batch descriptor; cu_q / cu_k are int32 device tensors (kept alive by the caller)."""
    return DsaBatch(len(cu_q) - 1, cu_q.data_ptr(), cu_k.data_ptr(), int(total_q), int(total_k), int(max_ctx))


def batch_of(p) -> DsaBatch:
    """Batch descriptor of a sparse_attention_03_amd.inputs.DSAInputs problem."""
    return make_batch(p.cu_q, p.cu_k, p.total_q, p.total_k, p.max_ctx)


def dsa_indexer_workspace_size(batch: DsaBatch, q_idx, act=DSA_ACT_RELU) -> int:
    n = _sz(0)
    _check(_lib.dsa_indexer_workspace_size(ctypes.byref(batch), _dtype_code(q_idx), q_idx.shape[1], q_idx.shape[2],
                                           act, ctypes.byref(n)), "dsa_indexer_workspace_size")
    return n.value


def dsa_indexer_scores(batch: DsaBatch, q_idx, k_idx, w, scores, act=DSA_ACT_RELU, ws=None, stream=None,
                       k_idx_scale=None):
    _check(_lib.dsa_indexer_scores(ctypes.byref(batch), _ptr(q_idx), _ptr(k_idx), _dtype_code(q_idx),
                                   _ptr(k_idx_scale), _ptr(w),
                                   q_idx.shape[1], q_idx.shape[2], act, _ptr(scores), scores.stride(0), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "dsa_indexer_scores")


def dsa_topk_workspace_size(batch: DsaBatch, k: int) -> int:
    n = _sz(0)
    _check(_lib.dsa_topk_workspace_size(ctypes.byref(batch), k, ctypes.byref(n)), "dsa_topk_workspace_size")
    return n.value


def dsa_topk(batch: DsaBatch, scores, k: int, idx, ws=None, stream=None):
    _check(_lib.dsa_topk(ctypes.byref(batch), _ptr(scores), scores.stride(0), k, _ptr(idx), _ptr(ws),
                         0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "dsa_topk")


def dsa_sparse_mla_attn_workspace_size(batch: DsaBatch, dtype: int, H: int, k: int, d_qk: int, d_v: int) -> int:
    n = _sz(0)
    _check(_lib.dsa_sparse_mla_attn_workspace_size(ctypes.byref(batch), dtype, H, k, d_qk, d_v, ctypes.byref(n)),
           "dsa_sparse_mla_attn_workspace_size")
    return n.value


def dsa_sparse_mla_attn(batch: DsaBatch, q, kv, idx, d_v: int, softmax_scale: float, out, lse=None, ws=None,
                        stream=None):
    _check(_lib.dsa_sparse_mla_attn(ctypes.byref(batch), _ptr(q), _ptr(kv), _dtype_code(q), _ptr(idx), idx.shape[1],
                                    q.shape[1], q.shape[2], d_v, float(softmax_scale), _ptr(out), _ptr(lse),
                                    _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "dsa_sparse_mla_attn")


def dsa_dense_mla_attn_workspace_size(batch: DsaBatch, dtype: int, H: int, d_qk: int, d_v: int) -> int:
    n = _sz(0)
    _check(_lib.dsa_dense_mla_attn_workspace_size(ctypes.byref(batch), dtype, H, d_qk, d_v, ctypes.byref(n)),
           "dsa_dense_mla_attn_workspace_size")
    return n.value


def dsa_dense_mla_attn(batch: DsaBatch, q, kv, d_v: int, softmax_scale: float, out, lse=None, ws=None, stream=None):
    _check(_lib.dsa_dense_mla_attn(ctypes.byref(batch), _ptr(q), _ptr(kv), _dtype_code(q), q.shape[1], q.shape[2],
                                   d_v, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "dsa_dense_mla_attn")


def forward_params(batch: DsaBatch, q_idx, k_idx, w, q, kv, k: int, d_v: int, softmax_scale: float, out,
                   lse=None, out_idx=None, act=DSA_ACT_RELU, q_block=0, k_idx_scale=None) -> DsaForwardParams:
    p = DsaForwardParams()
    p.batch = ctypes.pointer(batch)
    p.q_idx, p.k_idx, p.idx_dtype, p.w = q_idx.data_ptr(), k_idx.data_ptr(), _dtype_code(q_idx), w.data_ptr()
    p.k_idx_scale = None if k_idx_scale is None else k_idx_scale.data_ptr()
    p.H_I, p.d_I, p.act = q_idx.shape[1], q_idx.shape[2], act
    p.q, p.kv, p.dtype = q.data_ptr(), kv.data_ptr(), _dtype_code(q)
    p.H, p.d_qk, p.d_v, p.softmax_scale = q.shape[1], q.shape[2], d_v, float(softmax_scale)
    p.k, p.q_block = k, q_block
    p.out = out.data_ptr()
    p.lse = None if lse is None else lse.data_ptr()
    p.out_idx = None if out_idx is None else out_idx.data_ptr()
    return p


def dsa_sparse_mla_backward_workspace_size(batch: DsaBatch, H: int, k: int) -> int:
    n = _sz(0)
    _check(_lib.dsa_sparse_mla_backward_workspace_size(ctypes.byref(batch), H, k, ctypes.byref(n)),
           "dsa_sparse_mla_backward_workspace_size")
    return n.value


def dsa_sparse_mla_backward(batch: DsaBatch, q, kv, idx, d_v: int, softmax_scale: float, lse, dout, dq, dkv, ws,
                            stream=None):
    """Adds the sparse attention's gradients for dout into dq [total_q, H, d_qk] and dkv [total_k, d_qk]."""
    _check(_lib.dsa_sparse_mla_backward(ctypes.byref(batch), _ptr(q), _ptr(kv), _dtype_code(q), _ptr(idx),
                                        idx.shape[1], q.shape[1], q.shape[2], d_v, float(softmax_scale),
                                        _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dkv), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)), "dsa_sparse_mla_backward")


def dsa_attn_target(batch: DsaBatch, q, kv, softmax_scale: float, lse, p, idx=None, stream=None):
    """Alignment target p [total_q, ld_p] (dense when idx is None)."""
    _check(_lib.dsa_attn_target(ctypes.byref(batch), _ptr(q), _ptr(kv), _dtype_code(q), _ptr(idx),
                                0 if idx is None else idx.shape[1], q.shape[1], q.shape[2], float(softmax_scale),
                                _ptr(lse), _ptr(p), p.stride(0), _stream(stream)), "dsa_attn_target")


def dsa_indexer_kl(batch: DsaBatch, scores, p, loss=None, dI=None, idx=None, stream=None):
    _check(_lib.dsa_indexer_kl(ctypes.byref(batch), _ptr(scores), scores.stride(0), _ptr(idx),
                               0 if idx is None else idx.shape[1], _ptr(p), p.stride(0), _ptr(loss), _ptr(dI),
                               _stream(stream)), "dsa_indexer_kl")


def dsa_indexer_backward(batch: DsaBatch, q_idx, k_idx, w, g, dq_idx, dw, dk_idx, act=DSA_ACT_RELU, idx=None,
                         k_idx_scale=None, stream=None):
    """Adds the index score's gradients for the upstream g into dq_idx, dw, dk_idx."""
    _check(_lib.dsa_indexer_backward(ctypes.byref(batch), _ptr(q_idx), _ptr(k_idx), _dtype_code(q_idx),
                                     _ptr(k_idx_scale), _ptr(w), q_idx.shape[1], q_idx.shape[2], act, _ptr(idx),
                                     0 if idx is None else idx.shape[1], _ptr(g), g.stride(0), _ptr(dq_idx), _ptr(dw),
                                     _ptr(dk_idx), _stream(stream)), "dsa_indexer_backward")


def dsa_cache_append(k_new=None, k_cache=None, k_scale=None, kv_new=None, kv_cache=None, dst_rows=None,
                     stream=None):
    """New tokens into the caches: k_new [n, d_I] (fp32/bf16) -> k_cache [rows, d_I]
    (uint8 E4M3 codes) and k_scale [rows] (uint8 E8M0, optional); kv_new [n, d_qk]
    -> kv_cache [rows, d_qk]; dst_rows [n] int32 (None: token t -> row t)."""
    n = (k_new if k_new is not None else kv_new).shape[0]
    cache_rows = (k_cache if k_new is not None else kv_cache).shape[0]
    if k_new is not None and kv_new is not None:
        assert kv_new.shape[0] == n and kv_cache.shape[0] == cache_rows
    _check(_lib.dsa_cache_append(n, _ptr(dst_rows), cache_rows,
                                 _ptr(k_new), DSA_F32 if k_new is None else _dtype_code(k_new),
                                 0 if k_new is None else k_new.shape[1], _ptr(k_cache), _ptr(k_scale),
                                 _ptr(kv_new), DSA_BF16 if kv_new is None else _dtype_code(kv_new),
                                 0 if kv_new is None else kv_new.shape[1], _ptr(kv_cache), _stream(stream)),
           "dsa_cache_append")


def dsa_forward_workspace_size(params: DsaForwardParams) -> int:
    n = _sz(0)
    _check(_lib.dsa_forward_workspace_size(ctypes.byref(params), ctypes.byref(n)), "dsa_forward_workspace_size")
    return n.value


def dsa_forward(params: DsaForwardParams, ws, stream=None):
    _check(_lib.dsa_forward(ctypes.byref(params), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                            _stream(stream)), "dsa_forward")


def dsa_forward_noalloc(params: DsaForwardParams, stream=None):
    """dsa_forward on the library's static scratch (no workspace argument)."""
    _check(_lib.dsa_forward_noalloc(ctypes.byref(params), _stream(stream)), "dsa_forward_noalloc")


def version() -> str:
    return _lib.dsa_version().decode()
