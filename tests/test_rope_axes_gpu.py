"""GPU parity of the per-axis 3D RoPE form (sana_rope with a grid): the kernels
stage the t, h and w tables in LDS and derive each token's coordinates from its
position.  The angle values equal the full [pos][16] tables' entries, so every
entry point must give bit-identical results with either form, and match the
float64 oracle within the usual tolerances."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, inputs_on_device, to_dev, to_np, torch_mod
from metrics import check
from workloads import WORKLOADS, generate, reduced

pytestmark = pytest.mark.gpu


def _forms(grid, split=(8, 12, 12)):
    dev = device()
    return la.rope3d_device(*grid, dev, split=split), la.rope3d_axes_device(*grid, dev, split=split)


def _same(a, b, what):
    torch = torch_mod()
    ia, ib = (t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32) for t in (a, b))
    assert bool((ia == ib).all()), f"{what}: the two RoPE forms differ"


def _workload(grid, H, dtype="bf16", seed=0):
    return reduced(WORKLOADS["video720p_rope3d"], H=H, N=grid[0] * grid[1] * grid[2], grid=grid, dtype=dtype,
                   scale=0.5 if dtype == "bf16" else 1.0, seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_axes_equal_table(dtype):
    grid = (4, 10, 25)  # 1000 tokens: several tiles and a ragged tail
    w = _workload(grid, 6, dtype)
    print(f"case forward axes dtype={dtype}", flush=True)
    x = generate(w)
    q, k, v = inputs_on_device(x)
    table, axes = _forms(grid)
    o_t = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=table)
    o_a = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=axes)
    _same(o_a, o_t, "forward")
    check(to_np(o_a), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps, angles=oracle.rope3d_angles(*grid)),
          dtype, f"forward, per-axis RoPE ({dtype})")


def test_full_720p_layer_axes():
    """The SANA-Video 720p layer (21 x 22 x 40, 70 heads) with per-axis tables."""
    w = WORKLOADS["video720p_rope3d"]
    print("case full 720p per-axis RoPE", flush=True)
    x = generate(w)
    q, k, v = inputs_on_device(x)
    table, axes = _forms(w.grid)
    o_a = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=axes)
    _same(o_a, la.sana_linattn_forward(q, k, v, eps=w.eps, rope=table), "720p forward")
    check(to_np(o_a), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps,
                                     angles=oracle.rope3d_angles(*w.grid)), "bf16", "720p, per-axis RoPE")


def test_packed_layout_axes_equal_table():
    torch = torch_mod()
    grid = (3, 8, 20)
    w = _workload(grid, 4)
    print("case packed forward axes", flush=True)
    x = generate(w)
    buf = torch.empty(w.B, w.N, 3, w.H, w.D, dtype=torch.bfloat16, device=device())
    for i, n in enumerate(("q", "k", "v")):
        buf[:, :, i] = to_dev(x.raw[n], "bf16").permute(0, 2, 1, 3)
    q, k, v = (buf[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    table, axes = _forms(grid)
    outs = []
    for rope in (table, axes):
        o = torch.empty(w.B, w.N, w.H, w.D, dtype=torch.bfloat16, device=device()).permute(0, 2, 1, 3)
        la.sana_linattn_forward(q, k, v, o=o, eps=w.eps, rope=rope)
        outs.append(o)
    _same(outs[1], outs[0], "packed forward")


def test_block_calls_axes_equal_table():
    """The whole-sequence block-causal call, and one chunk through
    block_forward at a position offset after state_update of the chunks before
    it; then apply on the resulting state."""
    torch = torch_mod()
    grid = (6, 10, 12)   # 720 tokens, chunks of 2 frames = 240
    w = _workload(grid, 5)
    print("case block calls axes", flush=True)
    x = generate(w)
    q, k, v = inputs_on_device(x)
    table, axes = _forms(grid)
    res = {}
    for name, rope in (("table", table), ("axes", axes)):
        kv = torch.zeros(1, w.H, 32, 32, device=device())
        z = torch.zeros(1, w.H, 32, device=device())
        o_seq = la.sana_linattn_block_causal(q, k, v, 240, kv_out=kv, ksum_out=z, eps=w.eps, rope=rope)
        kv2 = torch.zeros_like(kv)
        z2 = torch.zeros_like(z)
        la.sana_linattn_state_update(k[:, :, :480].contiguous(), v[:, :, :480].contiguous(), kv2, z2, rope=rope.at(0))
        o_c = la.sana_linattn_block_forward(q[:, :, 480:].contiguous(), k[:, :, 480:].contiguous(),
                                            v[:, :, 480:].contiguous(), kv_in=kv2, ksum_in=z2, kv_out=kv2,
                                            ksum_out=z2, eps=w.eps, rope=rope.at(480))
        o_ap = la.sana_linattn_apply(q[:, :, 100:400].contiguous(), kv, z, eps=w.eps, rope=rope.at(100))
        res[name] = (o_seq, kv, z, o_c, kv2, z2, o_ap)
    for a, b, what in zip(res["axes"], res["table"], ("sequence", "kv", "z", "chunk", "kv2", "z2", "apply")):
        _same(a, b, what)
    ref, _, _ = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], 240, w.eps,
                                    angles=oracle.rope3d_angles(*grid))
    check(to_np(res["axes"][0]), ref, "bf16", "block-causal sequence, per-axis RoPE")


@pytest.mark.parametrize("dtype,chunk", [("bf16", None), ("bf16", 200), ("f32", None)])
def test_backward_axes_equal_table(dtype, chunk):
    grid = (4, 10, 20)
    w = _workload(grid, 3, dtype, seed=3)
    print(f"case backward axes dtype={dtype} chunk={chunk}", flush=True)
    x = generate(w, names=("q", "k", "v", "dout"))
    q, k, v = inputs_on_device(x)
    do = to_dev(x.raw["dout"], dtype)
    table, axes = _forms(grid)
    g_t = la.sana_linattn_backward(q, k, v, do, chunk=chunk, eps=w.eps, rope=table)
    g_a = la.sana_linattn_backward(q, k, v, do, chunk=chunk, eps=w.eps, rope=axes)
    for a, b, name in zip(g_a, g_t, ("dq", "dk", "dv")):
        _same(a, b, f"backward {name}")
    ref = oracle.backward(x.f64["q"], x.f64["k"], x.f64["v"], x.f64["dout"], w.eps,
                          angles=oracle.rope3d_angles(*grid), chunk=chunk)
    for got, want, name in zip(g_a, ref[:3], ("dq", "dk", "dv")):
        check(to_np(got), want, dtype, f"backward {name}, per-axis RoPE ({dtype}, chunk={chunk})")


def test_state_update_backward_axes_equal_table():
    torch = torch_mod()
    grid = (2, 12, 30)
    w = _workload(grid, 2)
    print("case state_update_backward axes", flush=True)
    x = generate(w)
    _, k, v = inputs_on_device(x)
    g = torch.Generator().manual_seed(9)
    dkv = torch.randn(1, w.H, 32, 32, generator=g).to(device())
    dz = torch.randn(1, w.H, 32, generator=g).to(device())
    table, axes = _forms(grid)
    r_t = la.sana_linattn_state_update_backward(k[:, :, 100:].contiguous(), v[:, :, 100:].contiguous(), dkv, dz,
                                                rope=table.at(100))
    r_a = la.sana_linattn_state_update_backward(k[:, :, 100:].contiguous(), v[:, :, 100:].contiguous(), dkv, dz,
                                                rope=axes.at(100))
    for a, b, name in zip(r_a, r_t, ("dk", "dv")):
        _same(a, b, f"state_update_backward {name}")


def test_other_split_axes_equal_table():
    """A split other than 8/12/12 (pairs 2/4/10), where a lane's four pairs
    cross an axis boundary in a different place."""
    grid = (5, 6, 7)
    split = (4, 8, 20)
    w = _workload(grid, 2)
    print("case split 4/8/20", flush=True)
    x = generate(w)
    q, k, v = inputs_on_device(x)
    table, axes = _forms(grid, split)
    o_t = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=table)
    o_a = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=axes)
    _same(o_a, o_t, "split 4/8/20")
    check(to_np(o_a), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps,
                                     angles=oracle.rope3d_angles(*grid, split=split)), "bf16", "split 4/8/20")
