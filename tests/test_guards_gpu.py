"""Canary guard bands around everything the kernels write.

Every output, state and workspace below sits inside a larger device buffer
whose 4 KiB before and after (and, for a strided output, the gaps between its
rows) hold a fixed byte pattern.  After each call the pattern must be intact bit
for bit, every input must be unchanged, and the results must equal those of the
same call on ordinary tensors bit for bit (which also checks that a call is
deterministic).  Shapes are ragged: several split partials per head, a partial
last tile, odd head counts."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
from gpu_util import device, torch_mod

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """`nbytes` of device memory with PATTERN bytes GUARD before and after."""

    def __init__(self, torch, nbytes):
        self.torch = torch
        self.n = int(nbytes)
        self.buf = torch.full((GUARD + self.n + GUARD,), PATTERN, dtype=torch.uint8, device=device())

    def bytes(self):
        return self.buf[GUARD:GUARD + self.n]

    def tensor(self, shape, dtype):
        return self.bytes().view(dtype).view(shape)

    def intact(self):
        t = self.torch
        return bool((self.buf[:GUARD] == PATTERN).all()) and bool((self.buf[GUARD + self.n:] == PATTERN).all())


def _guarded_like(torch, t, fill=None):
    g = Guarded(torch, t.numel() * t.element_size())
    x = g.tensor(tuple(t.shape), t.dtype)
    if fill is not None:
        x.copy_(fill)
    return g, x


def _same(torch, a, b):
    it = torch.int16 if a.dtype == torch.bfloat16 else (torch.int32 if a.element_size() == 4 else torch.uint8)
    return torch.equal(a.contiguous().view(it), b.contiguous().view(it))


def _inputs(torch, B, H, N, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return tuple((torch.randn(B, H, N, 32, generator=g) * 0.5).to(dt).to(device()) for _ in range(4))


def _state(torch, B, H, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(B, H, 32, 32, generator=g) * 0.1).to(device()), torch.rand(B, H, 32, generator=g).to(device())


def _check_inputs(torch, before, after):
    for a, b in zip(before, after):
        assert _same(torch, a, b), "an input changed"


@pytest.mark.parametrize("dtype,rope", [("bf16", None), ("bf16", "axes"), ("bf16", "table"), ("f32", None)])
def test_forward_guards(dtype, rope):
    torch = torch_mod()
    B, H, N = 1, 3, 2000 if rope is None else 5 * 8 * 50
    q, k, v, _ = _inputs(torch, B, H, N, dtype, 1)
    r = None
    if rope == "axes":
        r = la.rope3d_axes_device(5, 8, 50, device())
    elif rope == "table":
        r = la.rope3d_device(5, 8, 50, device())
    dt = la.SANA_DT_BF16 if dtype == "bf16" else la.SANA_DT_F32
    gw = Guarded(torch, la.workspace_bytes(B, H, N, dtype=dt, has_rope=r is not None))
    gw.bytes().fill_(0x5A)
    go, o = _guarded_like(torch, q)
    keep = [x.clone() for x in (q, k, v)]
    la.sana_linattn_forward(q, k, v, o=o, eps=1e-6, rope=r, workspace=gw.bytes())
    ref = la.sana_linattn_forward(q, k, v, eps=1e-6, rope=r)
    torch.cuda.synchronize()
    assert go.intact() and gw.intact(), "a guard band was written"
    _check_inputs(torch, keep, (q, k, v))
    assert _same(torch, o, ref)


def test_block_calls_guards():
    """block_forward (read-only and committing in place), block_causal, the
    allocation-free block_forward, state_update and apply."""
    torch = torch_mod()
    B, H, N = 1, 5, 1700
    q, k, v, _ = _inputs(torch, B, H, N, "bf16", 2)
    kv0, z0 = _state(torch, B, H, 3)
    keep = [x.clone() for x in (q, k, v)]

    gw = Guarded(torch, la.workspace_bytes(B, H, N))
    gkv, kv = _guarded_like(torch, kv0, kv0)
    gz, z = _guarded_like(torch, z0, z0)
    go, o = _guarded_like(torch, q)
    la.sana_linattn_block_forward(q, k, v, o=o, kv_in=kv, ksum_in=z, eps=1e-6, workspace=gw.bytes())
    assert _same(torch, kv, kv0) and _same(torch, z, z0), "a read-only call changed the state"
    la.sana_linattn_block_forward(q, k, v, o=o, kv_in=kv, ksum_in=z, kv_out=kv, ksum_out=z, eps=1e-6,
                                  workspace=gw.bytes())
    kv_r, z_r = kv0.clone(), z0.clone()
    o_r = la.sana_linattn_block_forward(q, k, v, kv_in=kv_r, ksum_in=z_r, kv_out=kv_r, ksum_out=z_r, eps=1e-6)
    torch.cuda.synchronize()
    assert all(g.intact() for g in (gw, gkv, gz, go))
    assert _same(torch, o, o_r) and _same(torch, kv, kv_r) and _same(torch, z, z_r)

    # the allocation-free form writes only its outputs and states
    gkv2, kv2 = _guarded_like(torch, kv0, kv0)
    gz2, z2 = _guarded_like(torch, z0, z0)
    go2, o2 = _guarded_like(torch, q)
    la.sana_linattn_block_forward_noalloc(q, k, v, o=o2, kv_in=kv2, ksum_in=z2, kv_out=kv2, ksum_out=z2, eps=1e-6)
    torch.cuda.synchronize()
    assert all(g.intact() for g in (gkv2, gz2, go2))
    assert _same(torch, o2, o_r) and _same(torch, kv2, kv_r)

    # a whole sequence in chunks of 400 (a ragged last chunk)
    gwc = Guarded(torch, la.block_causal_workspace_bytes(B, H, N, 400))
    gkv3, kv3 = _guarded_like(torch, kv0, kv0)
    gz3, z3 = _guarded_like(torch, z0, z0)
    go3, o3 = _guarded_like(torch, q)
    la.sana_linattn_block_causal(q, k, v, 400, o=o3, kv_in=kv3, ksum_in=z3, kv_out=kv3, ksum_out=z3, eps=1e-6,
                                 workspace=gwc.bytes())
    kv_c, z_c = kv0.clone(), z0.clone()
    o_c = la.sana_linattn_block_causal(q, k, v, 400, kv_in=kv_c, ksum_in=z_c, kv_out=kv_c, ksum_out=z_c, eps=1e-6)
    torch.cuda.synchronize()
    assert all(g.intact() for g in (gwc, gkv3, gz3, go3))
    assert _same(torch, o3, o_c) and _same(torch, kv3, kv_c) and _same(torch, z3, z_c)

    # state_update, then apply on that state
    gkv4, kv4 = _guarded_like(torch, kv0, kv0)
    gz4, z4 = _guarded_like(torch, z0, z0)
    gw4 = Guarded(torch, la.workspace_bytes(B, H, N))
    la.sana_linattn_state_update(k, v, kv4, z4, workspace=gw4.bytes())
    go5, o5 = _guarded_like(torch, q)
    la.sana_linattn_apply(q, kv4, z4, o=o5, eps=1e-6)
    torch.cuda.synchronize()
    assert all(g.intact() for g in (gkv4, gz4, gw4, go5))
    assert _same(torch, kv4, kv_r) and _same(torch, z4, z_r)
    assert _same(torch, o5, o_r)
    _check_inputs(torch, keep, (q, k, v))


def test_strided_forward_guards():
    """Q, K, V read from a packed [B, N, 3, H, D] buffer and O written into a
    [B, N, H, D] view whose rows leave gaps: the gaps hold the pattern too."""
    torch = torch_mod()
    B, H, N = 1, 4, 1500
    q, k, v, _ = _inputs(torch, B, H, N, "bf16", 4)
    buf = torch.empty(B, N, 3, H, 32, dtype=torch.bfloat16, device=device())
    for j, t in enumerate((q, k, v)):
        buf[:, :, j] = t.permute(0, 2, 1, 3)
    qv, kv_, vv = (buf[:, :, j].permute(0, 2, 1, 3) for j in range(3))
    # O as every other head slot of a [B, N, 2H, D] region: heads at even slots
    g = Guarded(torch, B * N * 2 * H * 32 * 2)
    region = g.tensor((B, N, 2 * H, 32), torch.bfloat16)
    o = region[:, :, 0::2].permute(0, 2, 1, 3)
    gw = Guarded(torch, la.workspace_bytes(B, H, N))
    la.sana_linattn_forward(qv, kv_, vv, o=o, eps=1e-6, workspace=gw.bytes())
    ref = la.sana_linattn_forward(q, k, v, eps=1e-6)
    torch.cuda.synchronize()
    assert g.intact() and gw.intact()
    gaps = region[:, :, 1::2].contiguous().view(torch.uint8)
    assert bool((gaps == PATTERN).all()), "a store landed between the output's rows"
    assert _same(torch, o, ref)


@pytest.mark.parametrize("chunk", [None, 600])
def test_backward_guards(chunk):
    torch = torch_mod()
    B, H, N = 1, 3, 1300
    q, k, v, do = _inputs(torch, B, H, N, "bf16", 5)
    kv0, z0 = _state(torch, B, H, 6)
    dkv_o, dz_o = _state(torch, B, H, 7)
    L = N if chunk is None else chunk
    gw = Guarded(torch, la.backward_workspace_bytes(B, H, N, L))
    outs = [_guarded_like(torch, q) for _ in range(3)]
    gdkv, dkv_in = _guarded_like(torch, kv0)
    gdz, dz_in = _guarded_like(torch, z0)
    keep = [x.clone() for x in (q, k, v, do, kv0, z0, dkv_o, dz_o)]
    # the forward leaves its chunk states in the workspace for the saved-state backward
    if chunk is None:
        la.sana_linattn_block_forward(q, k, v, kv_in=kv0, ksum_in=z0, eps=1e-6, workspace=gw.bytes())
    else:
        la.sana_linattn_block_causal(q, k, v, chunk, kv_in=kv0, ksum_in=z0, eps=1e-6, workspace=gw.bytes())
    la.sana_linattn_backward_saved(q, k, v, do, gw.bytes(), chunk=chunk, dq=outs[0][1], dk=outs[1][1],
                                   dv=outs[2][1], dkv_out=dkv_o, dksum_out=dz_o, dkv_in=dkv_in, dksum_in=dz_in,
                                   eps=1e-6)
    ref = la.sana_linattn_backward(q, k, v, do, chunk=chunk, kv_in=kv0, ksum_in=z0, dkv_out=dkv_o, dksum_out=dz_o,
                                   eps=1e-6)
    torch.cuda.synchronize()
    assert gw.intact() and gdkv.intact() and gdz.intact() and all(g.intact() for g, _ in outs)
    for (_, got), want in zip(outs, ref):
        assert _same(torch, got, want)
    _check_inputs(torch, keep, (q, k, v, do, kv0, z0, dkv_o, dz_o))


@pytest.mark.parametrize("rope", [False, True])
def test_projection_guards(rope):
    torch = torch_mod()
    B, H, N, C = 1, 3, 900, 96
    gen = torch.Generator().manual_seed(8)
    x = (torch.randn(B, N, C, generator=gen) * 0.5).to(torch.bfloat16).to(device())
    wk, wv, wq = ((torch.randn(H * 32, C, generator=gen) / C ** 0.5).to(torch.bfloat16).to(device())
                  for _ in range(3))
    r = la.rope3d_axes_device(9, 10, 10, device()) if rope else None
    kv0, z0 = _state(torch, B, H, 9)
    gkv, kv = _guarded_like(torch, kv0, kv0)
    gz, z = _guarded_like(torch, z0, z0)
    gw = Guarded(torch, la.project_state_workspace_bytes(B, H, N, C))
    la.sana_linattn_project_state(x, wk, wv, kv, z, rope=r, workspace=gw.bytes())
    kv_r, z_r = kv0.clone(), z0.clone()
    la.sana_linattn_project_state(x, wk, wv, kv_r, z_r, rope=r)
    go, o = _guarded_like(torch, torch.empty(B, H, N, 32, dtype=torch.bfloat16, device=device()))
    la.sana_linattn_project_apply(x, wq, kv_r, z_r, o=o, rope=r)
    o_r = la.sana_linattn_project_apply(x, wq, kv_r, z_r, rope=r)
    torch.cuda.synchronize()
    assert gkv.intact() and gz.intact() and gw.intact() and go.intact()
    assert _same(torch, kv, kv_r) and _same(torch, z, z_r) and _same(torch, o, o_r)


def test_temporal_conv_guards():
    torch = torch_mod()
    B, F, S, C = 1, 3, 130, 48
    gen = torch.Generator().manual_seed(10)
    x = (torch.randn(B, F, S, C, generator=gen) * 0.5).to(torch.bfloat16).to(device())
    w = (torch.randn(C, 3, generator=gen) * 0.3).to(device())
    b = (torch.randn(C, generator=gen) * 0.1).to(device())
    prev = (torch.randn(B, S, C, generator=gen) * 0.5).to(torch.bfloat16).to(device())
    gc, cache = _guarded_like(torch, prev, prev)
    gy, y = _guarded_like(torch, x)
    la.sana_linattn_temporal_conv3(x, w, b, cache_in=cache, cache_out=cache, y=y)
    cache_r = prev.clone()
    y_r = la.sana_linattn_temporal_conv3(x, w, b, cache_in=cache_r, cache_out=cache_r)
    torch.cuda.synchronize()
    assert gc.intact() and gy.intact()
    assert _same(torch, y, y_r) and _same(torch, cache, cache_r)
    assert np.array_equal(cache.view(torch.int16).cpu().numpy(), x[:, -1].contiguous().view(torch.int16).cpu().numpy())
