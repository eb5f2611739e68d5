"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library (``sparse_attention_03_amd``)
never does, and this package imports nothing from the library.

Thin ctypes wrapper over ``liboracle.so`` (plain C, double precision, built by
``oracle/build.py``).  Element formats are passed as raw storage:
``float32`` arrays, ``uint16`` bfloat16 bit patterns, or ``uint8`` OCP E4M3FN
codes, with the matching dtype code.
"""
import ctypes
import os

import numpy as np

F32, BF16, FP8_E4M3 = 0, 1, 2
ACT_RELU, ACT_GELU = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_ORACLE_LIB: another build of the oracle (e.g. the sanitized build)
_LIB_PATH = os.environ.get("DSA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.dsa_oracle_e4m3_value.argtypes = [i32]
        L.dsa_oracle_e4m3_value.restype = dbl
        L.dsa_oracle_indexer.argtypes = [i32, p, p, i32, p, p, p, i32, p, p, i32, i32, i32, p, i64]
        L.dsa_oracle_topk.argtypes = [i32, p, p, i32, p, p, i64, i32, p]
        L.dsa_oracle_sparse_mla.argtypes = [i32, p, p, i32, p, p, p, i32, p, i32, i32, i32, i32, dbl, p, p]
        L.dsa_oracle_dense_mla.argtypes = [i32, p, p, i32, p, p, p, i32, i32, i32, i32, dbl, p, p]
        L.dsa_oracle_quantize_keys.argtypes = [p, i32, i64, i32, i32, p, p]
        L.dsa_oracle_sparse_mla_backward.argtypes = [i32, p, p, i32, p, p, p, i32, p, i32, i32, i32, i32, dbl,
                                                     p, p, p]
        L.dsa_oracle_attn_target.argtypes = [i32, p, p, i32, p, p, p, i32, p, i32, i32, i32, dbl, p]
        L.dsa_oracle_indexer_kl.argtypes = [i32, i32, p, p, p, p, p]
        L.dsa_oracle_indexer_backward.argtypes = [i32, p, p, i32, p, p, p, i32, p, p, i32, i32, i32, p, i32, p,
                                                  p, p, p]
        L.dsa_oracle_forward.argtypes = [i32, p, p, i32, p, p, p, i32, p, p, i32, i32, i32,
                                         p, p, i32, i32, i32, i32, dbl, i32, i64, p, p, p, p]
        for f in (L.dsa_oracle_indexer, L.dsa_oracle_topk, L.dsa_oracle_sparse_mla, L.dsa_oracle_dense_mla,
                  L.dsa_oracle_quantize_keys, L.dsa_oracle_forward, L.dsa_oracle_attn_target,
                  L.dsa_oracle_indexer_kl, L.dsa_oracle_indexer_backward, L.dsa_oracle_sparse_mla_backward):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8_E4M3
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def _rows(rows, cu_q):
    if rows is None:
        return np.arange(int(cu_q[-1]), dtype=np.int32)
    return _c(rows, np.int32)


def e4m3_value(code: int) -> float:
    return lib().dsa_oracle_e4m3_value(int(code))


def indexer(cu_q, cu_k, q_idx, k_idx, w, act=ACT_RELU, ld=None, rows=None, k_scale=None):
    """Scores [nrows, ld] float64; entries s > pos are left at 0.  `k_scale`:
    optional E8M0 byte per key row (FP8 keys scaled by 2^(byte - 127))."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q_idx, k_idx = np.ascontiguousarray(q_idx), np.ascontiguousarray(k_idx)
    dt = _dtype_code(q_idx)
    assert _dtype_code(k_idx) == dt
    nrows, H_I, d_I = q_idx.shape
    assert nrows == len(rows) and k_idx.shape[1] == d_I
    w = _c(w, np.float32)
    assert w.shape == (nrows, H_I)
    if ld is None:
        ld = int(np.max(np.diff(cu_k)))
    if k_scale is not None:
        k_scale = _c(k_scale, np.uint8)
        assert k_scale.shape == (k_idx.shape[0],)
    out = np.zeros((nrows, ld), dtype=np.float64)
    rc = lib().dsa_oracle_indexer(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows),
                                  _ptr(q_idx), _ptr(k_idx), dt, _ptr(k_scale), _ptr(w), H_I, d_I, act,
                                  _ptr(out), ld)
    if rc != 0:
        raise ValueError("oracle indexer: invalid batch / rows")
    return out


def topk(cu_q, cu_k, scores, k, rows=None):
    """Selected positions [nrows, k] int32, ascending, -1 padded."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    scores = _c(scores, np.float32)
    nrows, ld = scores.shape
    assert nrows == len(rows)
    idx = np.empty((nrows, k), dtype=np.int32)
    rc = lib().dsa_oracle_topk(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows),
                               _ptr(scores), ld, k, _ptr(idx))
    if rc != 0:
        raise ValueError("oracle topk: invalid batch / rows")
    return idx


def sparse_mla(cu_q, cu_k, q, kv, idx, d_v, scale, rows=None):
    """(out [nrows, H, d_v] float64, lse [nrows, H] float64)."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q, kv = np.ascontiguousarray(q), np.ascontiguousarray(kv)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt
    nrows, H, d_qk = q.shape
    assert nrows == len(rows) and kv.shape[1] == d_qk
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    out = np.zeros((nrows, H, d_v), dtype=np.float64)
    lse = np.zeros((nrows, H), dtype=np.float64)
    rc = lib().dsa_oracle_sparse_mla(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows),
                                     _ptr(q), _ptr(kv), dt, _ptr(idx), k, H, d_qk, d_v, float(scale),
                                     _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle sparse_mla: invalid batch / rows / indices")
    return out, lse


def sparse_mla_backward(cu_q, cu_k, q, kv, idx, d_v, scale, dout, rows=None):
    """Gradients of the sparse MQA attention for the upstream dout [nrows, H, d_v]:
    (dq [nrows, H, d_qk], dkv [total_k, d_qk]) float64, dkv summed over rows."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q, kv = np.ascontiguousarray(q), np.ascontiguousarray(kv)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt
    nrows, H, d_qk = q.shape
    idx = _c(idx, np.int32)
    dout = _c(dout, np.float64)
    assert dout.shape == (nrows, H, d_v)
    dq = np.zeros((nrows, H, d_qk), dtype=np.float64)
    dkv = np.zeros(kv.shape, dtype=np.float64)
    rc = lib().dsa_oracle_sparse_mla_backward(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows), _ptr(q),
                                              _ptr(kv), dt, _ptr(idx), idx.shape[1], H, d_qk, d_v, float(scale),
                                              _ptr(dout), _ptr(dq), _ptr(dkv))
    if rc != 0:
        raise ValueError("oracle sparse_mla_backward: invalid batch / rows / indices")
    return dq, dkv


def dense_mla(cu_q, cu_k, q, kv, d_v, scale, rows=None):
    """Dense causal MQA over every candidate [0, pos] (the masked mode of short
    prefill): (out [nrows, H, d_v] float64, lse [nrows, H] float64)."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q, kv = np.ascontiguousarray(q), np.ascontiguousarray(kv)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt
    nrows, H, d_qk = q.shape
    assert nrows == len(rows) and kv.shape[1] == d_qk
    out = np.zeros((nrows, H, d_v), dtype=np.float64)
    lse = np.zeros((nrows, H), dtype=np.float64)
    rc = lib().dsa_oracle_dense_mla(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows),
                                    _ptr(q), _ptr(kv), dt, H, d_qk, d_v, float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle dense_mla: invalid batch / rows")
    return out, lse


def quantize_keys(src, scaled=False):
    """Indexer keys [n, d] (float32, or bfloat16 bits as uint16) to E4M3FN codes
    [n, d] uint8, plus E8M0 per-row scales [n] uint8 when `scaled`."""
    src = np.ascontiguousarray(src)
    dt = _dtype_code(src)
    n, d = src.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    scale = np.zeros(n if scaled else 1, dtype=np.uint8)
    rc = lib().dsa_oracle_quantize_keys(_ptr(src), dt, n, d, int(scaled), _ptr(codes), _ptr(scale))
    if rc != 0:
        raise ValueError("oracle quantize_keys: source must be float32 or bfloat16")
    return (codes, scale) if scaled else codes


def attn_target(cu_q, cu_k, q, kv, scale, idx=None, ld=None, rows=None):
    """Indexer-alignment target p [nrows, m] float64: the main attention's
    per-head probabilities over each row's candidates, summed over heads and
    L1-normalised.  idx None: dense, entry e = position e (m = ld, default the
    longest context); else entry e = position idx[i, e] (m = k)."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q, kv = np.ascontiguousarray(q), np.ascontiguousarray(kv)
    dt = _dtype_code(q)
    assert _dtype_code(kv) == dt
    nrows, H, d_qk = q.shape
    if idx is not None:
        idx = _c(idx, np.int32)
        m = idx.shape[1]
    else:
        m = int(np.max(np.diff(cu_k))) if ld is None else ld
    out = np.zeros((nrows, m), dtype=np.float64)
    rc = lib().dsa_oracle_attn_target(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows), _ptr(q), _ptr(kv),
                                      dt, _ptr(idx), m, H, d_qk, float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle attn_target: invalid batch / rows")
    return out


def indexer_kl(I, p, cnt):
    """(loss [nrows], dI [nrows, m]) of KL(p || softmax(I)) over each row's first
    cnt[i] entries."""
    I, p = _c(I, np.float64), _c(p, np.float64)
    cnt = _c(cnt, np.int32)
    nrows, m = I.shape
    loss = np.zeros(nrows, dtype=np.float64)
    dI = np.zeros((nrows, m), dtype=np.float64)
    if lib().dsa_oracle_indexer_kl(nrows, m, _ptr(cnt), _ptr(I), _ptr(p), _ptr(loss), _ptr(dI)) != 0:
        raise ValueError("oracle indexer_kl: bad counts")
    return loss, dI


def indexer_backward(cu_q, cu_k, q_idx, k_idx, w, g, act=ACT_RELU, idx=None, rows=None, k_scale=None):
    """(dq_idx [nrows, H_I, d_I], dw [nrows, H_I], dk_idx [total_k, d_I]) float64
    for the upstream gradient g [nrows, m] over each row's candidates (dense:
    entry e = position e; else entry e = position idx[i, e])."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q_idx, k_idx = np.ascontiguousarray(q_idx), np.ascontiguousarray(k_idx)
    dt = _dtype_code(q_idx)
    assert _dtype_code(k_idx) == dt
    nrows, H_I, d_I = q_idx.shape
    w = _c(w, np.float32)
    g = _c(g, np.float64)
    m = g.shape[1]
    if idx is not None:
        idx = _c(idx, np.int32)
        assert idx.shape == g.shape
    if k_scale is not None:
        k_scale = _c(k_scale, np.uint8)
    dq = np.zeros((nrows, H_I, d_I), dtype=np.float64)
    dw = np.zeros((nrows, H_I), dtype=np.float64)
    dk = np.zeros(k_idx.shape, dtype=np.float64)
    rc = lib().dsa_oracle_indexer_backward(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows), _ptr(q_idx),
                                           _ptr(k_idx), dt, _ptr(k_scale), _ptr(w), H_I, d_I, act, _ptr(idx), m,
                                           _ptr(g), _ptr(dq), _ptr(dw), _ptr(dk))
    if rc != 0:
        raise ValueError("oracle indexer_backward: invalid batch / rows")
    return dq, dw, dk


def forward(cu_q, cu_k, q_idx, k_idx, w, q, kv, k, d_v, scale, act=ACT_RELU, rows=None, ld=None, k_scale=None):
    """Indexer -> fp32 rounding -> top-k -> sparse attention.

    Returns (out, lse, scores_f32, idx)."""
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _rows(rows, cu_q)
    q_idx, k_idx, q, kv = (np.ascontiguousarray(a) for a in (q_idx, k_idx, q, kv))
    nrows, H_I, d_I = q_idx.shape
    _, H, d_qk = q.shape
    w = _c(w, np.float32)
    if k_scale is not None:
        k_scale = _c(k_scale, np.uint8)
    if ld is None:
        ld = int(np.max(np.diff(cu_k)))
    out = np.zeros((nrows, H, d_v), dtype=np.float64)
    lse = np.zeros((nrows, H), dtype=np.float64)
    sc = np.zeros((nrows, ld), dtype=np.float32)
    idx = np.empty((nrows, k), dtype=np.int32)
    rc = lib().dsa_oracle_forward(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), nrows, _ptr(rows),
                                  _ptr(q_idx), _ptr(k_idx), _dtype_code(q_idx), _ptr(k_scale), _ptr(w), H_I, d_I, act,
                                  _ptr(q), _ptr(kv), _dtype_code(q), H, d_qk, d_v, float(scale), k, ld,
                                  _ptr(out), _ptr(lse), _ptr(sc), _ptr(idx))
    if rc != 0:
        raise ValueError("oracle forward failed")
    return out, lse, sc, idx
