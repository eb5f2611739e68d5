"""dsa_forward_noalloc (the forward on the library's static scratch) through
the C interface, against dsa_forward on a caller workspace: two calls in a row
on one device, the second with a smaller batch, each bit-identical to
dsa_forward; a batch larger than the scratch is refused before any launch."""
import pytest
import torch

from dsa_check import announce
from sparse_attention_03_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCRATCH_BYTES = 128 << 20


def _noalloc(p):
    from sparse_attention_03_amd import libdsa as L
    b = L.batch_of(p)
    out = torch.empty((p.total_q, p.H, p.d_v), dtype=p.q.dtype, device=DEV)
    lse = torch.empty((p.total_q, p.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((p.total_q, p.k), dtype=torch.int32, device=DEV)
    prm = L.forward_params(b, p.q_idx, p.k_idx, p.w, p.q, p.kv, p.k, p.d_v, p.scale, out, lse, idx,
                           q_block=p.q_block)
    need = L.dsa_forward_workspace_size(prm)
    L.dsa_forward_noalloc(prm)
    torch.cuda.synchronize()
    return out, lse, idx, need


def test_noalloc_forward_equals_forward_twice():
    from sparse_attention_03_amd import dsa
    # decode steps: 16 sequences of 20000 tokens, k = 2048 (key splits, a
    # segmented top-k), then a smaller one: 8 sequences of 5000 tokens, k = 512
    problems = [gen.make_problem("noalloc", [20000] * 16, [1] * 16, H_I=64, H=128, k=2048, device=DEV, seed=41),
                gen.make_problem("noalloc", [5000] * 8, [1] * 8, H_I=64, H=128, k=512, device=DEV, seed=42)]
    needs = []
    for i, p in enumerate(problems):
        announce("forward_noalloc call", i, "rows", p.total_q)
        out, lse, idx, need = _noalloc(p)
        needs.append(need)
        assert 0 < need <= SCRATCH_BYTES
        out_r, lse_r, idx_r = dsa.Forward(p)()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_r)
        assert torch.equal(out, out_r) and torch.equal(lse, lse_r)
    assert needs[1] < needs[0]


def test_noalloc_forward_refuses_a_batch_beyond_the_scratch():
    from sparse_attention_03_amd import libdsa as L
    announce("forward_noalloc too large")
    # an 8192-token prefill in one 8192-row chunk: 8192 x 8192 fp32 scores alone are 256 MiB
    p = gen.make_problem("noalloc", [8192], [8192], H_I=64, H=128, k=2048, device=DEV, seed=43, q_block=8192)
    out = torch.full((p.total_q, p.H, p.d_v), 7.0, dtype=p.q.dtype, device=DEV)
    b = L.batch_of(p)
    prm = L.forward_params(b, p.q_idx, p.k_idx, p.w, p.q, p.kv, p.k, p.d_v, p.scale, out, q_block=8192)
    assert L.dsa_forward_workspace_size(prm) > SCRATCH_BYTES
    with pytest.raises(L.DsaError) as e:
        L.dsa_forward_noalloc(prm)
    assert e.value.status == L.DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)      # nothing was enqueued
