"""The allocation-free block_forward (sana_linattn_block_forward_noalloc)
against the workspace entry point it mirrors, called through the C ABI: the
same kernels on the same geometry, so outputs and commits must agree bit for
bit.  Two calls in a row share the GPU's static scratch array, the second with
a smaller input."""

import ctypes

import pytest

import linear_attention_diffusion_amd as la
from gpu_util import device, torch_mod

pytestmark = pytest.mark.gpu


def _bits(torch, t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _case(torch, gen, B, H, N, commit, rope_grid=None):
    dev = device()
    q, k, v = ((torch.randn(B, H, N, 32, generator=gen) * 0.5).to(torch.bfloat16).to(dev) for _ in range(3))
    kv0 = (torch.randn(B, H, 32, 32, generator=gen) * 0.1).to(dev)
    z0 = torch.rand(B, H, 32, generator=gen).to(dev)
    rope = la.rope3d_axes_device(*rope_grid, dev) if rope_grid else None

    # the workspace entry point
    kv_ref, z_ref = kv0.clone(), z0.clone()
    o_ref = la.sana_linattn_block_forward(q, k, v, kv_in=kv_ref, ksum_in=z_ref,
                                          kv_out=kv_ref if commit else None, ksum_out=z_ref if commit else None,
                                          rope=rope)
    # the allocation-free one, straight through the C ABI
    kv, z = kv0.clone(), z0.clone()
    o = torch.empty_like(q)
    P = ctypes.c_void_p
    rc = la.lib().sana_linattn_block_forward_noalloc(
        P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), P(kv.data_ptr()), P(z.data_ptr()),
        P(kv.data_ptr()) if commit else None, P(z.data_ptr()) if commit else None, B, H, N, 32, la.SANA_DT_BF16,
        ctypes.c_float(1e-6), None if rope is None else ctypes.byref(rope.struct()),
        P(torch.cuda.current_stream(dev).cuda_stream))
    assert rc == la.SANA_OK, la.sana_linattn_status_string(rc)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch, o), _bits(torch, o_ref)), f"outputs differ (B={B}, H={H}, N={N})"
    assert torch.equal(_bits(torch, kv), _bits(torch, kv_ref)) and torch.equal(_bits(torch, z), _bits(torch, z_ref))
    if not commit:
        assert torch.equal(kv, kv0) and torch.equal(z, z0), "a read-only call changed the state"


def test_noalloc_equals_block_forward_on_two_calls():
    torch = torch_mod()
    gen = torch.Generator().manual_seed(21)
    # several split partials per head and a ragged last split, committing in place
    _case(torch, gen, B=1, H=6, N=3000, commit=True)
    # then a smaller call on the same scratch: fewer heads and tokens, read-only, 3D RoPE
    _case(torch, gen, B=1, H=2, N=700, commit=False, rope_grid=(7, 10, 10))


def test_noalloc_chunk_loop_matches():
    """A block-causal loop of three chunks committing after each, as in
    inference, against the same loop through the workspace entry point."""
    torch = torch_mod()
    dev = device()
    gen = torch.Generator().manual_seed(22)
    B, H, L = 1, 4, 1100
    ref_kv, ref_z = torch.zeros(B, H, 32, 32, device=dev), torch.zeros(B, H, 32, device=dev)
    kv, z = torch.zeros_like(ref_kv), torch.zeros_like(ref_z)
    for _ in range(3):
        q, k, v = ((torch.randn(B, H, L, 32, generator=gen) * 0.5).to(torch.bfloat16).to(dev) for _ in range(3))
        o_ref = la.sana_linattn_block_forward(q, k, v, kv_in=ref_kv, ksum_in=ref_z, kv_out=ref_kv, ksum_out=ref_z)
        o = la.sana_linattn_block_forward_noalloc(q, k, v, kv_in=kv, ksum_in=z, kv_out=kv, ksum_out=z)
        assert torch.equal(_bits(torch, o), _bits(torch, o_ref))
    assert torch.equal(kv, ref_kv) and torch.equal(z, ref_z)
