"""The C interface without a GPU: the library loads, exports every entry point
the header declares, and rejects invalid calls on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libdsa.h")


@pytest.fixture(scope="module")
def L():
    lib = os.path.join(ROOT, "sparse_attention_03_amd", "lib", "libdsa.so")
    if not os.path.exists(lib):
        from sparse_attention_03_amd import build
        build.build()
    from sparse_attention_03_amd import libdsa
    return libdsa


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_forward"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(L.EXPORTED)


def test_status_strings_and_version(L):
    assert L._lib.dsa_status_string(L.DSA_OK) == b"DSA_OK"
    assert L._lib.dsa_status_string(L.DSA_ERR_WORKSPACE) == b"DSA_ERR_WORKSPACE"
    assert L.version().startswith("libdsa")


class FakeTensor:
    """Just enough of a tensor for the binding: a pointer, a shape, a dtype."""

    def __init__(self, ptr, shape, dtype, stride0=None):
        import torch
        self._ptr, self.shape, self.dtype = ptr, shape, dtype
        self._stride0 = stride0 if stride0 is not None else (shape[1] if len(shape) > 1 else 1)
        self._torch = torch

    def data_ptr(self):
        return self._ptr

    def stride(self, i):
        return self._stride0

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return 1


def _batch(L, cu=0x1000, total_q=8, total_k=8, max_ctx=8, nseq=1):
    b = L.DsaBatch(nseq, cu, cu + 0x100, total_q, total_k, max_ctx)
    return b


def _call_indexer(L, b, q=0x10000, k=0x20000, w=0x30000, s=0x40000, H_I=64, d_I=128, dt=2, act=0, ld=64, ks=None):
    return L._lib.dsa_indexer_scores(ctypes.byref(b), q, k, dt, ks, w, H_I, d_I, act, s, ld, 0x50000, 1 << 20, None)


def test_indexer_validation(L):
    b = _batch(L)
    assert _call_indexer(L, b, q=0) == L.DSA_ERR_INVALID_ARG
    assert b"NULL" in L._lib.dsa_last_error()
    assert _call_indexer(L, b, q=0x10004) == L.DSA_ERR_INVALID_ARG        # misaligned
    assert _call_indexer(L, b, d_I=136) == L.DSA_ERR_UNSUPPORTED          # fp8: d_I up to 128 ...
    assert _call_indexer(L, b, d_I=24) == L.DSA_ERR_UNSUPPORTED           # ... a multiple of 16
    assert _call_indexer(L, b, H_I=18) == L.DSA_ERR_UNSUPPORTED           # fp8: H_I a multiple of 4
    assert _call_indexer(L, b, H_I=68) == L.DSA_ERR_UNSUPPORTED           # ... up to 64
    assert _call_indexer(L, b, dt=1) == L.DSA_ERR_UNSUPPORTED             # bf16 indexer
    assert _call_indexer(L, b, act=7) == L.DSA_ERR_INVALID_ARG
    assert _call_indexer(L, b, ld=4) == L.DSA_ERR_INVALID_ARG             # ld < max_ctx
    assert _call_indexer(L, b, ld=66) == L.DSA_ERR_INVALID_ARG            # ld % 4
    assert _call_indexer(L, _batch(L, nseq=0)) == L.DSA_ERR_INVALID_ARG
    assert _call_indexer(L, _batch(L, cu=0)) == L.DSA_ERR_INVALID_ARG
    assert _call_indexer(L, _batch(L, max_ctx=9)) == L.DSA_ERR_INVALID_ARG  # > total_k
    assert _call_indexer(L, _batch(L, total_q=9)) == L.DSA_ERR_INVALID_ARG  # more queries than keys
    assert _call_indexer(L, b, dt=0, H_I=8, d_I=32, ks=0x60000) == L.DSA_ERR_INVALID_ARG  # scales need FP8 keys
    assert L._lib.dsa_indexer_scores(None, 0x10000, 0x20000, 2, None, 0x30000, 64, 128, 0, 0x40000, 64, None, 0,
                                     None) == L.DSA_ERR_INVALID_ARG
    # FP8 + ReLU keeps 528 bytes per query row in the workspace; GELU and F32 need none
    f = L._lib.dsa_indexer_scores
    assert f(ctypes.byref(b), 0x10000, 0x20000, 2, None, 0x30000, 64, 128, 0, 0x40000, 64, None, 0, None) \
        == L.DSA_ERR_WORKSPACE
    assert f(ctypes.byref(b), 0x10000, 0x20000, 2, None, 0x30000, 64, 128, 0, 0x40000, 64, 0x50000, 100, None) \
        == L.DSA_ERR_WORKSPACE
    n = ctypes.c_size_t(123)
    assert L._lib.dsa_indexer_workspace_size(ctypes.byref(b), 2, 64, 128, 0, ctypes.byref(n)) == L.DSA_OK
    assert n.value >= 8 * 528 and n.value % 256 == 0
    assert L._lib.dsa_indexer_workspace_size(ctypes.byref(b), 2, 64, 128, 1, ctypes.byref(n)) == L.DSA_OK
    assert n.value == 0
    assert L._lib.dsa_indexer_workspace_size(ctypes.byref(b), 0, 8, 32, 0, ctypes.byref(n)) == L.DSA_OK
    assert n.value == 0
    assert L._lib.dsa_indexer_workspace_size(ctypes.byref(b), 2, 18, 128, 0, ctypes.byref(n)) == L.DSA_ERR_UNSUPPORTED


def test_topk_validation(L):
    b = _batch(L)
    f = L._lib.dsa_topk
    assert f(ctypes.byref(b), 0x40000, 64, 0, 0x50000, None, 0, None) == L.DSA_ERR_UNSUPPORTED     # k = 0
    assert f(ctypes.byref(b), 0x40000, 64, 4096, 0x50000, None, 0, None) == L.DSA_ERR_UNSUPPORTED  # k > 2048
    assert f(ctypes.byref(b), 0x40000, 64, 32, 0, None, 0, None) == L.DSA_ERR_INVALID_ARG
    assert f(ctypes.byref(b), 0, 64, 32, 0x50000, None, 0, None) == L.DSA_ERR_INVALID_ARG
    n = ctypes.c_size_t(123)
    assert L._lib.dsa_topk_workspace_size(ctypes.byref(b), 32, ctypes.byref(n)) == L.DSA_OK and n.value == 0


def test_attention_validation(L):
    b = _batch(L)
    f = L._lib.dsa_sparse_mla_attn

    def call(q=0x10000, kv=0x20000, dt=1, idx=0x30000, k=32, H=128, dqk=576, dv=512, scale=0.1, out=0x40000):
        return f(ctypes.byref(b), q, kv, dt, idx, k, H, dqk, dv, scale, out, None, None, 0, None)

    assert call(q=0) == L.DSA_ERR_INVALID_ARG
    assert call(out=0x40008) == L.DSA_ERR_INVALID_ARG
    assert call(dqk=600) == L.DSA_ERR_UNSUPPORTED    # bf16: d_qk up to 576 ...
    assert call(dqk=568, dv=64) == L.DSA_ERR_UNSUPPORTED  # ... a multiple of 16
    assert call(dqk=576, dv=520) == L.DSA_ERR_UNSUPPORTED  # d_v up to 512
    # narrower bf16 shapes pass validation (here they stop at the missing device)
    assert call(dqk=512, dv=128) not in (L.DSA_ERR_UNSUPPORTED, L.DSA_ERR_INVALID_ARG)
    assert call(H=100) == L.DSA_ERR_UNSUPPORTED    # bf16 heads: multiples of 8 up to 128
    assert call(H=136) == L.DSA_ERR_UNSUPPORTED
    assert call(dt=2) == L.DSA_ERR_UNSUPPORTED
    assert call(k=3000) == L.DSA_ERR_UNSUPPORTED
    assert call(dv=600) == L.DSA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == L.DSA_ERR_INVALID_ARG
    assert call(dt=0, dqk=2048) == L.DSA_ERR_UNSUPPORTED


def test_cache_append_validation(L):
    f = L._lib.dsa_cache_append

    def call(n=4, dst=None, rows=16, kn=0x10000, kdt=0, dI=128, kc=0x20000, ks=None, vn=0x30000, vdt=1, dqk=576,
             vc=0x40000):
        return f(n, dst, rows, kn, kdt, dI, kc, ks, vn, vdt, dqk, vc, None)

    assert call(n=-1) == L.DSA_ERR_INVALID_ARG
    assert call(rows=-1) == L.DSA_ERR_INVALID_ARG
    assert call(kdt=2) == L.DSA_ERR_UNSUPPORTED              # keys come in as F32 or BF16
    assert call(dI=96) == L.DSA_ERR_UNSUPPORTED
    assert call(kc=0) == L.DSA_ERR_INVALID_ARG
    assert call(kn=0x10008) == L.DSA_ERR_INVALID_ARG         # k_new 16-byte aligned
    assert call(kc=0x20004) == L.DSA_ERR_INVALID_ARG         # k_cache 8-byte aligned
    assert call(kn=None, ks=0x50000) == L.DSA_ERR_INVALID_ARG
    assert call(vdt=2) == L.DSA_ERR_UNSUPPORTED
    assert call(dqk=100) == L.DSA_ERR_INVALID_ARG            # 200-byte rows: not a multiple of 16
    assert call(vc=0) == L.DSA_ERR_INVALID_ARG
    assert call(vn=0x30008) == L.DSA_ERR_INVALID_ARG
    assert call(n=1 << 40) == L.DSA_ERR_UNSUPPORTED           # latent part beyond 2^31 chunks
    # nothing to do: no device call
    assert call(n=0) == L.DSA_OK
    assert call(kn=None, vn=None) == L.DSA_OK


def test_alignment_and_backward_validation(L):
    b = _batch(L)
    # dsa_attn_target(batch, q, kv, dtype, idx, k, H, d_qk, scale, lse, p, ld_p, stream)
    t = L._lib.dsa_attn_target
    assert t(ctypes.byref(b), 0x10000, 0x20000, 1, None, 0, 128, 576, 0.1, None, 0x40000, 32, None) \
        == L.DSA_ERR_INVALID_ARG                                          # lse NULL
    assert t(ctypes.byref(b), 0x10000, 0x20000, 1, None, 0, 128, 576, 0.1, 0x30000, 0x40000, 4, None) \
        == L.DSA_ERR_INVALID_ARG                                          # ld_p below whole tiles of max_ctx
    assert t(ctypes.byref(b), 0x10000, 0x20000, 1, 0x50000, 100, 128, 576, 0.1, 0x30000, 0x40000, 100, None) \
        == L.DSA_ERR_INVALID_ARG                                          # ld_p below k rounded up to 32
    assert t(ctypes.byref(b), 0x10000, 0x20000, 1, None, 0, 100, 576, 0.1, 0x30000, 0x40000, 32, None) \
        == L.DSA_ERR_UNSUPPORTED                                          # H
    assert t(ctypes.byref(b), 0x10000, 0x20000, 1, None, 0, 128, 512, 0.1, 0x30000, 0x40000, 32, None) \
        == L.DSA_ERR_UNSUPPORTED                                          # bf16 target: d_qk = 576 only
    # dsa_indexer_kl(batch, scores, ld_s, idx, k, p, ld_p, loss, dI, stream)
    k = L._lib.dsa_indexer_kl
    assert k(ctypes.byref(b), 0x10000, 64, None, 0, 0, 64, None, None, None) == L.DSA_ERR_INVALID_ARG   # p NULL
    assert k(ctypes.byref(b), 0x10000, 64, None, 0, 0x20008, 64, None, None, None) == L.DSA_ERR_INVALID_ARG
    assert k(ctypes.byref(b), 0x10000, 64, None, 0, 0x20000, 4, None, None, None) == L.DSA_ERR_INVALID_ARG
    assert k(ctypes.byref(b), 0x10000, 64, 0x30000, 0, 0x20000, 64, None, None, None) == L.DSA_ERR_INVALID_ARG
    assert k(ctypes.byref(b), 0x10000, 2, None, 0, 0x20000, 64, None, None, None) == L.DSA_ERR_INVALID_ARG
    # dsa_indexer_backward(batch, q_idx, k_idx, dtype, k_scale, w, H_I, d_I, act, idx, k, g, ld_g, dq, dw, dk, stream)
    bw = L._lib.dsa_indexer_backward

    def ib(dt=2, g=0x40000, ld=64, dq=0x50000, idx=None, kk=0, H_I=64):
        return bw(ctypes.byref(b), 0x10000, 0x20000, dt, None, 0x30000, H_I, 128 if dt == 2 else 32, 0, idx, kk,
                  g, ld, dq, 0x60000, 0x70000, None)
    assert ib(dt=0, H_I=8) == L.DSA_ERR_UNSUPPORTED                  # FP8 only
    assert bw(ctypes.byref(b), 0x10000, 0x20000, 2, None, 0x30000, 64, 64, 0, None, 0, 0x40000, 64, 0x50000,
              0x60000, 0x70000, None) == L.DSA_ERR_UNSUPPORTED       # d_I = 128 only
    assert ib(g=0) == L.DSA_ERR_INVALID_ARG
    assert ib(dq=0x50004) == L.DSA_ERR_INVALID_ARG                   # misaligned gradient
    assert ib(ld=4) == L.DSA_ERR_INVALID_ARG                         # ld_g < max_ctx
    assert ib(idx=0x80000, kk=0) == L.DSA_ERR_INVALID_ARG            # k < 1 with idx
    # dsa_sparse_mla_backward(batch, q, kv, dtype, idx, k, H, d_qk, d_v, scale, lse, dout, dq, dkv, ws, ws_bytes, s)
    ab = L._lib.dsa_sparse_mla_backward

    def mb(dt=1, lse=0x30000, dout=0x40000, dkv=0x60000, ws=0x70000, wsb=1 << 30, H=128):
        return ab(ctypes.byref(b), 0x10000, 0x20000, dt, 0x80000, 64, H, 576 if dt == 1 else 64, 512 if dt == 1 else 64,
                  0.1, lse, dout, 0x50000, dkv, ws, wsb, None)
    assert mb(dt=0) == L.DSA_ERR_UNSUPPORTED                         # BF16 only
    assert mb(lse=None) == L.DSA_ERR_INVALID_ARG
    assert mb(dout=0x40004) == L.DSA_ERR_INVALID_ARG
    assert mb(dkv=None) == L.DSA_ERR_INVALID_ARG
    assert mb(ws=None) == L.DSA_ERR_WORKSPACE
    assert mb(wsb=16) == L.DSA_ERR_WORKSPACE
    assert mb(H=96) == L.DSA_ERR_UNSUPPORTED
    assert ab(ctypes.byref(b), 0x10000, 0x20000, 1, 0x80000, 64, 128, 512, 256, 0.1, 0x30000, 0x40000, 0x50000,
              0x60000, 0x70000, 1 << 30, None) == L.DSA_ERR_UNSUPPORTED   # backward: 576 / 512 only
    n = ctypes.c_size_t(0)
    assert L._lib.dsa_sparse_mla_backward_workspace_size(ctypes.byref(b), 128, 64, ctypes.byref(n)) == L.DSA_OK
    assert n.value == 4 * ((8 * 128 * 64 * 2 + 255) // 256 * 256)
    assert L._lib.dsa_sparse_mla_backward_workspace_size(ctypes.byref(b), 100, 64, ctypes.byref(n)) \
        == L.DSA_ERR_UNSUPPORTED


def test_forward_validation(L):
    import torch
    b = _batch(L)
    t8 = FakeTensor(0x10000, (8, 64, 128), torch.float8_e4m3fn)
    k8 = FakeTensor(0x20000, (8, 128), torch.float8_e4m3fn)
    w = FakeTensor(0x30000, (8, 64), torch.float32)
    q = FakeTensor(0x40000, (8, 128, 576), torch.bfloat16)
    kv = FakeTensor(0x50000, (8, 576), torch.bfloat16)
    out = FakeTensor(0x60000, (8, 128, 512), torch.bfloat16)
    p = L.forward_params(b, t8, k8, w, q, kv, 2048, 512, 0.07, out)
    p.q_block = -1
    assert L._lib.dsa_forward(ctypes.byref(p), None, 0, None) == L.DSA_ERR_INVALID_ARG
    p.q_block = 0
    p.d_v = 500
    assert L._lib.dsa_forward(ctypes.byref(p), None, 0, None) == L.DSA_ERR_UNSUPPORTED
    p.d_v = 512
    p.idx_dtype = 0
    p.H_I, p.d_I = 8, 32
    p.k_idx_scale = 0x70000
    assert L._lib.dsa_forward(ctypes.byref(p), None, 0, None) == L.DSA_ERR_INVALID_ARG   # scales need FP8 keys
    p.idx_dtype, p.H_I, p.d_I, p.k_idx_scale = 2, 64, 128, None
    p.w = 0
    assert L._lib.dsa_forward(ctypes.byref(p), None, 0, None) == L.DSA_ERR_INVALID_ARG
    assert L._lib.dsa_forward(None, None, 0, None) == L.DSA_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert L._lib.dsa_forward_workspace_size(ctypes.byref(p), None) == L.DSA_ERR_INVALID_ARG
