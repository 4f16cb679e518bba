"""GPU parity of the two-launch chunk call: with dense bf16 layouts, one chunk
split a few ways and a few dozen heads (the 480p video chunk of the
block-causal loop, B1 H70 N4680), the state pass leaves each head's partials
and the head's apply workgroups, on one XCD, each sum them onto the carried
state themselves before applying it: no finalize launch.  They sum in the
finalize's order, so a padded-row view of the same inputs (64 elements between
tokens), which takes the three-launch path (state pass, finalize, apply), must
give the same outputs, saved state and commit bit for bit.  Both are also held
to the oracle at the bf16 bar ("SANA-Video" paper notes 2.3: the chunk's
queries see the carried state plus the whole chunk)."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, to_dev, to_np, torch_mod
from metrics import check
from workloads import WORKLOADS, generate, reduced

pytestmark = pytest.mark.gpu


def _padded(t):
    torch = torch_mod()
    buf = torch.zeros(*t.shape[:3], 64, dtype=t.dtype, device=t.device)
    buf[..., :32] = t
    return buf[..., :32]


def _same(a, b, what):
    torch = torch_mod()
    assert a.shape == b.shape
    ia, ib = (t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32) for t in (a, b))
    n = int((ia != ib).sum())
    assert n == 0, f"{what}: {n} elements differ from the three-launch path"


def _carried(B, H, seed):
    torch = torch_mod()
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, H, 32, 32, generator=g) * 20, torch.rand(B, H, 32, generator=g) * 200


# (B, H, N): the 480p chunk (3 parts per head, 7 splits, a short last split and
# part), 4 splits of 256 tokens with a short last one, 36 heads at 4 parts each
# with a part past the last token, 32 heads (the fewest that take the path) at
# 12 splits, 128 heads (2 parts per head), two batches of 20 heads, and heads
# long enough (over 8192 tokens) for the 8-wave workgroups, 8 parts per head
CASES = [(1, 70, 4680), (1, 70, 1000), (1, 36, 520), (1, 32, 3001), (2, 64, 2000), (2, 20, 777), (1, 40, 9000)]


@pytest.mark.parametrize("B,H,N", CASES)
@pytest.mark.parametrize("mode", ["commit_in_place", "first_chunk", "read_only", "commit_elsewhere"])
def test_fold_block_forward_equals_three_launch_path(B, H, N, mode):
    torch = torch_mod()
    assert la.forward_launches(B, H, N) == 2, "shape meant to take the two-launch path"
    w = reduced(WORKLOADS["video480p_blockcausal"], B=B, H=H, N=N, mode="noncausal")
    print(f"case folded block_forward B={B} H={H} N={N} mode={mode}", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    kv0, z0 = _carried(B, H, N)
    results = []
    for view in (lambda t: t, _padded):
        ws = la.make_workspace(B, H, N, device())
        ws.fill_(0x5A)
        kv_in, z_in = kv0.to(device()), z0.to(device())
        if mode == "first_chunk":
            kv_in = z_in = None
            kv_out, z_out = torch.full((B, H, 32, 32), 7.0, device=device()), torch.full((B, H, 32), 7.0,
                                                                                           device=device())
        elif mode == "commit_in_place":
            kv_out, z_out = kv_in, z_in
        elif mode == "commit_elsewhere":
            kv_out, z_out = torch.empty_like(kv_in), torch.empty_like(z_in)
        else:
            kv_out = z_out = None
        o = la.sana_linattn_block_forward(view(q), view(k), view(v), kv_in=kv_in, ksum_in=z_in, kv_out=kv_out,
                                          ksum_out=z_out, eps=w.eps, workspace=ws)
        torch.cuda.synchronize()
        results.append((o, kv_out, z_out, kv_in, z_in))
    (o, kv_a, z_a, kin_a, zin_a), (o2, kv_b, z_b, kin_b, zin_b) = results
    _same(o, o2, "O")
    if kv_a is not None:
        _same(kv_a, kv_b, "committed S")
        _same(z_a, z_b, "committed z")
    if mode != "first_chunk":
        # the carried state is untouched unless committed in place
        if mode != "commit_in_place":
            _same(kin_a, kv0.to(device()), "carried S")
            _same(zin_a, z0.to(device()), "carried z")
    S0 = np.zeros((B, H, 32, 32)) if mode == "first_chunk" else kv0.double().numpy()
    Z0 = np.zeros((B, H, 32)) if mode == "first_chunk" else z0.double().numpy()
    ref_o, ref_s, ref_z = oracle.block_forward(x.f64["q"], x.f64["k"], x.f64["v"], S0, Z0, w.eps)
    check(to_np(o), ref_o, "bf16", f"folded block_forward {mode}")
    if kv_a is not None:
        check(to_np(kv_a), ref_s, "f32", "folded committed S")
        check(to_np(z_a), ref_z, "f32", "folded committed z")


def test_fold_chunk_loop_480p_full_size():
    """Three chunks of the 480p loop at full size (H70, 4680 tokens each), each
    committing in place, against the oracle's block-causal form and against
    the same loop through padded views (three-launch path), bit for bit."""
    torch = torch_mod()
    w0 = WORKLOADS["video480p_blockcausal"]
    w = reduced(w0, N=3 * w0.chunk)
    print(f"case folded chunk loop H={w.H} chunk={w.chunk} chunks=3", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    res = []
    for view in (lambda t: t, _padded):
        kv = torch.zeros(1, w.H, 32, 32, device=device())
        z = torch.zeros(1, w.H, 32, device=device())
        outs = []
        for c in range(3):
            sl = slice(c * w.chunk, (c + 1) * w.chunk)
            qc, kc, vc = (t[:, :, sl].contiguous() for t in (q, k, v))
            outs.append(la.sana_linattn_block_forward(view(qc), view(kc), view(vc), kv_in=kv if c else None,
                                                      ksum_in=z if c else None, kv_out=kv, ksum_out=z, eps=w.eps))
        res.append((torch.cat(outs, dim=2), kv, z))
    _same(res[0][0], res[1][0], "O")
    _same(res[0][1], res[1][1], "S")
    _same(res[0][2], res[1][2], "z")
    ref, S, Z = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], w.chunk, w.eps)
    check(to_np(res[0][0]), ref, "bf16", "folded 480p chunk loop")
    check(to_np(res[0][1]), S, "f32", "folded 480p final S")
    check(to_np(res[0][2]), Z, "f32", "folded 480p final z")


def test_fold_saved_state_serves_backward():
    """The workspace keeps the chunk state for backward_saved, as the
    three-launch path leaves it: gradients equal the recomputing backward bit for bit."""
    torch = torch_mod()
    B, H, N = 1, 40, 1500
    assert la.forward_launches(B, H, N) == 2
    w = reduced(WORKLOADS["video480p_blockcausal"], H=H, N=N, mode="noncausal")
    print(f"case folded forward + backward_saved H={H} N={N}", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    g = torch.Generator(device=device()).manual_seed(3)
    do = torch.randn(B, H, N, 32, generator=g, device=device()).to(torch.bfloat16)
    ws = la.make_workspace(B, H, N, device())
    la.sana_linattn_forward(q, k, v, eps=w.eps, workspace=ws)
    saved = la.sana_linattn_backward_saved(q, k, v, do, workspace=ws, eps=w.eps)
    fresh = la.sana_linattn_backward(q, k, v, do, eps=w.eps)
    for a, b, name in zip(saved[:3], fresh[:3], ("dq", "dk", "dv")):
        _same(a, b, name)


def test_fold_forward_4096px_full_size():
    """The Sana-1.6B 4096 px layer (B1 H70 N16384, 8-wave workgroups, 7 parts
    per head) through the forward, against the padded-view three-launch path
    bit for bit and against the oracle."""
    w = WORKLOADS["sana16b_4096px"]
    assert la.forward_launches(w.B, w.H, w.N) == 2
    print(f"case folded forward B={w.B} H={w.H} N={w.N}", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    o = la.sana_linattn_forward(q, k, v, eps=w.eps)
    o2 = la.sana_linattn_forward(_padded(q), _padded(k), _padded(v), eps=w.eps)
    _same(o, o2, "O")
    check(to_np(o), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps), "bf16", "folded 4096 px forward")


@pytest.mark.parametrize("B,H,N,grid,offset,commit", [(1, 70, 2 * 40 * 50, (2, 40, 50), 0, False),
                                                      (1, 40, 3 * 30 * 52, (5, 30, 52), 1560, True)])
def test_fold_per_axis_rope_equals_three_launch_path(B, H, N, grid, offset, commit):
    """SANA-Video's per-axis 3D RoPE ("SANA-Video" paper notes 2.2; section 3
    Stage 2) through the two-launch path: a forward over two latent frames,
    and a committing chunk call at a frame offset from a carried state, each
    bit for bit as the padded-view three-launch path and within the oracle
    bars."""
    torch = torch_mod()
    assert la.forward_launches(B, H, N, rope_form=2) == 2
    w = reduced(WORKLOADS["video720p_rope3d"], B=B, H=H, N=N, grid=grid, mode="rope")
    print(f"case folded per-axis RoPE B={B} H={H} N={N} offset={offset} commit={commit}", flush=True)
    x = generate(w)
    q, k, v = (to_dev(x.raw[n], "bf16") for n in ("q", "k", "v"))
    r = la.rope3d_axes_device(*grid, device()).at(offset)
    kv0, z0 = _carried(B, H, 11)
    res = []
    for view in (lambda t: t, _padded):
        if commit:
            kv, z = kv0.to(device()), z0.to(device())
            o = la.sana_linattn_block_forward(view(q), view(k), view(v), kv_in=kv, ksum_in=z, kv_out=kv, ksum_out=z,
                                              eps=w.eps, rope=r)
            res.append((o, kv, z))
        else:
            res.append((la.sana_linattn_forward(view(q), view(k), view(v), eps=w.eps, rope=r), None, None))
    _same(res[0][0], res[1][0], "O")
    ang = oracle.rope3d_angles(*grid)
    if commit:
        _same(res[0][1], res[1][1], "committed S")
        _same(res[0][2], res[1][2], "committed z")
        ref_o, ref_s, ref_z = oracle.block_forward(x.f64["q"], x.f64["k"], x.f64["v"], kv0.double().numpy(),
                                                   z0.double().numpy(), w.eps, ang, offset)
        check(to_np(res[0][0]), ref_o, "bf16", "folded RoPE block_forward")
        check(to_np(res[0][1]), ref_s, "f32", "folded RoPE committed S")
    else:
        check(to_np(res[0][0]), oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps, angles=ang), "bf16",
              "folded RoPE forward")
