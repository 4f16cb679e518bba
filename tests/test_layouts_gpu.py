"""GPU parity through strided layout views (the *_strided entry points, reached
from the binding with non-contiguous [B, H, N, D] views): Q, K, V read from a
packed [B, N, 3, H, D] projection-style buffer, outputs written to
[B, N, H, D].  Results must equal the contiguous calls bit for bit (the same
arithmetic in the same order) and the oracle within the usual tolerances."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, rope_for, to_dev, to_np, torch_mod
from metrics import check
from workloads import WORKLOADS, Workload, generate, reduced

pytestmark = pytest.mark.gpu


def _packed(x, names=("q", "k", "v")):
    """Contiguous [B, H, N, D] device tensors and [B, H, N, D] views of one
    packed [B, N, len(names), H, D] buffer holding the same values."""
    torch = torch_mod()
    w = x.workload
    flat = [to_dev(x.raw[n], w.dtype) for n in names]
    buf = torch.empty(w.B, w.N, len(names), w.H, w.D, dtype=flat[0].dtype, device=device())
    for i, t in enumerate(flat):
        buf[:, :, i] = t.permute(0, 2, 1, 3)
    views = [buf[:, :, i].permute(0, 2, 1, 3) for i in range(len(names))]
    assert not views[0].is_contiguous()
    return flat, views


def _bnhd(w, dtype):
    torch = torch_mod()
    return torch.empty(w.B, w.N, w.H, w.D, dtype=dtype, device=device()).permute(0, 2, 1, 3)


def _same(a, b):
    torch = torch_mod()
    assert a.shape == b.shape
    ia, ib = (t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32) for t in (a, b))
    assert bool((ia == ib).all())


@pytest.mark.parametrize("dtype,rope", [("bf16", False), ("bf16", True), ("f32", False), ("f32", True)])
def test_forward_packed_inputs(dtype, rope):
    base = WORKLOADS["video720p_rope3d"]
    w = reduced(base, H=6, N=4 * 10 * 25, grid=(4, 10, 25), mode="rope" if rope else "noncausal", dtype=dtype,
                scale=0.5 if dtype == "bf16" else 1.0)
    print(f"case forward packed dtype={dtype} rope={rope}", flush=True)
    x = generate(w)
    (q, k, v), (qv, kv_, vv) = _packed(x)
    r = rope_for(w) if rope else None
    o_ref = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=r)
    o = _bnhd(w, q.dtype)
    la.sana_linattn_forward(qv, kv_, vv, o=o, eps=w.eps, rope=r)
    _same(o, o_ref)
    ang = oracle.rope3d_angles(*w.grid) if rope else None
    check(to_np(o), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps, angles=ang), dtype, "packed forward")


@pytest.mark.parametrize("H", [5, 6])
def test_block_causal_and_block_forward_packed(H):
    """H = 5 takes the split-wave path (pairs would straddle batches), H = 6
    the whole-line kernels; N is ragged against every tile size."""
    torch = torch_mod()
    w = reduced(WORKLOADS["video480p_blockcausal"], H=H, N=3 * 700 + 111, chunk=700)
    print(f"case block-causal packed H={H}", flush=True)
    x = generate(w)
    (q, k, v), (qv, kv_, vv) = _packed(x)
    kv0 = torch.zeros(w.B, w.H, 32, 32, device=device())
    z0 = torch.zeros(w.B, w.H, 32, device=device())
    kv1, z1 = kv0.clone(), z0.clone()
    o_ref = la.sana_linattn_block_causal(q, k, v, w.chunk, kv_out=kv0, ksum_out=z0, eps=w.eps)
    o = _bnhd(w, q.dtype)
    la.sana_linattn_block_causal(qv, kv_, vv, w.chunk, o=o, kv_out=kv1, ksum_out=z1, eps=w.eps)
    _same(o, o_ref)
    _same(kv1, kv0)
    ref, _, _ = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], w.chunk, w.eps)
    check(to_np(o), ref, "bf16", "packed block_causal")
    # one chunk through block_forward with packed views (chunk 1's tokens)
    s, e = w.chunk, 2 * w.chunk
    kv2, z2 = torch.zeros_like(kv0), torch.zeros_like(z0)
    la.sana_linattn_state_update(k[:, :, :s].contiguous(), v[:, :, :s].contiguous(), kv2, z2)
    oc = la.sana_linattn_block_forward(qv[:, :, s:e], kv_[:, :, s:e], vv[:, :, s:e], kv_in=kv2, ksum_in=z2, eps=w.eps)
    _same(oc, o_ref[:, :, s:e])


@pytest.mark.parametrize("rope,grid,eps", [(False, (3, 8, 20), 1e-6), (True, (3, 8, 20), 1e-6),
                                           (False, (3, 7, 21), 1e-6), (True, (3, 7, 21), 1e-6),
                                           (False, (3, 7, 21), 0.0), ("axes", (2, 9, 25), 1e-6)])
def test_backward_packed(rope, grid, eps):
    """The backward read from a packed [B, N, 4, H, D] buffer (q, k, v, dO) and
    written to [B, N, H, D]: with H even the query and key passes take head
    pairs from whole lines; bit-identical to the contiguous call."""
    w = reduced(WORKLOADS["video720p_rope3d"], H=4, N=grid[0] * grid[1] * grid[2], grid=grid,
                mode="rope" if rope else "noncausal", eps=eps)
    print(f"case backward packed rope={rope} grid={grid} eps={eps}", flush=True)
    x = generate(w, names=("q", "k", "v", "dout"))
    (q, k, v, do), (qv, kv_, vv, dov) = _packed(x, ("q", "k", "v", "dout"))
    r = (la.rope3d_axes_device(*grid, device()) if rope == "axes" else rope_for(w)) if rope else None
    ref_dev = la.sana_linattn_backward(q, k, v, do, chunk=160, eps=w.eps, rope=r)
    outs = [_bnhd(w, q.dtype) for _ in range(3)]
    la.sana_linattn_backward(qv, kv_, vv, dov, chunk=160, dq=outs[0], dk=outs[1], dv=outs[2], eps=w.eps, rope=r)
    for a, b in zip(outs, ref_dev):
        _same(a, b)
    ang = oracle.rope3d_angles(*w.grid) if rope else None
    ref = oracle.backward(x.f64["q"], x.f64["k"], x.f64["v"], x.f64["dout"], w.eps, angles=ang, chunk=160)
    for got, want, name in zip(outs, ref[:3], ("dq", "dk", "dv")):
        check(to_np(got), want, "bf16", f"packed backward {name}")


def test_full_size_packed_forward():
    """The Sana-1.6B 4096 px layer read straight from a packed QKV buffer."""
    w = WORKLOADS["sana16b_4096px"]
    print("case full-size packed forward", flush=True)
    x = generate(w)
    (q, k, v), (qv, kv_, vv) = _packed(x)
    o = _bnhd(w, q.dtype)
    la.sana_linattn_forward(qv, kv_, vv, o=o, eps=w.eps)
    check(to_np(o), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps), "bf16", "full-size packed")
