"""GPU parity of the whole-head forward: with dense bf16 layouts and one chunk
of one split per head (short sequences over many heads, such as the Sana-0.6B
1024 px layer, B4 H36 N1024), a head's state and its apply run in one
workgroup and one launch.  A padded-row view of the same inputs (64 elements
between tokens) takes the two-pass path through the same arithmetic, so
outputs and committed states must agree bit for bit; both are also held to the
oracle at the bf16 bar."""

import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, to_dev, to_np, torch_mod
from metrics import check
from workloads import WORKLOADS, generate, reduced

pytestmark = pytest.mark.gpu


def _padded(t):
    """The values of contiguous [B, H, N, 32] t in a [B, H, N, 32] view with
    64 elements between tokens."""
    torch = torch_mod()
    buf = torch.zeros(*t.shape[:3], 64, dtype=t.dtype, device=t.device)
    buf[..., :32] = t
    view = buf[..., :32]
    assert not view.is_contiguous()
    return view


def _same(a, b):
    torch = torch_mod()
    assert a.shape == b.shape
    ia, ib = (t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32) for t in (a, b))
    assert bool((ia == ib).all())


@pytest.mark.parametrize("rope", [False, True])
def test_whole_head_forward_equals_two_pass(rope):
    w = reduced(WORKLOADS["sana06b_1024px"], mode="rope" if rope else "noncausal", grid=(4, 16, 16) if rope else None)
    print(f"case whole-head forward B={w.B} H={w.H} N={w.N} rope={rope}", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    r = la.rope3d_axes_device(*w.grid, device()) if rope else None
    o = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=r)
    o2 = la.sana_linattn_forward(_padded(q), _padded(k), _padded(v), eps=w.eps, rope=r)
    _same(o, o2)
    ang = oracle.rope3d_angles(*w.grid) if rope else None
    check(to_np(o), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps, angles=ang), "bf16", "whole-head forward")


@pytest.mark.parametrize("rope,offset", [(False, 0), (True, 37)])
def test_whole_head_block_forward_commits_like_two_pass(rope, offset):
    """A 200-token chunk (one split per head at any head count) from a carried
    state, committed in place, with RoPE at a position offset."""
    torch = torch_mod()
    w = reduced(WORKLOADS["video480p_blockcausal"], H=5, N=200, mode="noncausal")
    print(f"case whole-head block_forward H={w.H} N={w.N} rope={rope} offset={offset}", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    g = torch.Generator().manual_seed(5)
    kv0 = torch.randn(w.B, w.H, 32, 32, generator=g)
    z0 = torch.rand(w.B, w.H, 32, generator=g) * 50
    grid = (3, 8, 10)
    r = la.rope3d_axes_device(*grid, device()).at(offset) if rope else None
    kv_a, z_a = kv0.to(device()), z0.to(device())
    o = la.sana_linattn_block_forward(q, k, v, kv_in=kv_a, ksum_in=z_a, kv_out=kv_a, ksum_out=z_a, eps=w.eps, rope=r)
    kv_b, z_b = kv0.to(device()), z0.to(device())
    o2 = la.sana_linattn_block_forward(_padded(q), _padded(k), _padded(v), kv_in=kv_b, ksum_in=z_b, kv_out=kv_b,
                                       ksum_out=z_b, eps=w.eps, rope=r)
    _same(o, o2)
    _same(kv_a, kv_b)
    _same(z_a, z_b)
    ang = oracle.rope3d_angles(*grid) if rope else None
    ref_o, ref_s, ref_z = oracle.block_forward(x.f64["q"], x.f64["k"], x.f64["v"], kv0.double().numpy(),
                                               z0.double().numpy(), w.eps, ang, offset)
    check(to_np(o), ref_o, "bf16", "whole-head block_forward")
    check(to_np(kv_a), ref_s, "f32", "whole-head committed S")
    check(to_np(z_a), ref_z, "f32", "whole-head committed z")
