"""GPU parity of the backward (sana_linattn_backward, through the C ABI) against
the float64 oracle's backward on the same seeded inputs, element by element.

Q, K, V are the forward's draws and dO is drawn after them from the same
stream.  dQ, dK, dV use the forward's tolerances (bf16: rel-L2 <= 4e-3 and
floored max rel err <= 2e-2; fp32: rel-L2 <= 1e-5); the fp32 gradient of the
carried state is held to rel-L2 <= 1e-5 for fp32 inputs and 1e-4 for bf16
inputs (fp32 sums over up to ~50k tokens)."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, rope_for, split_chunks, to_dev, to_np, torch_mod
from metrics import check, rel_l2
from workloads import WORKLOADS, Workload, generate, reduced

pytestmark = pytest.mark.gpu


def _state_like(w, seed):
    """A realistic carried state: the state of another seeded draw of the same
    workload, rounded to fp32 (the values both sides then use)."""
    other = generate(w, seed=seed)
    S, z = oracle.kv_state(other.f64["k"], other.f64["v"])
    return S.astype(np.float32), z.astype(np.float32)


def _run(w, chunk, rope=False, carried=False, out_grad=False, seed=None, label=""):
    torch = torch_mod()
    print(f"case {label}: B={w.B} H={w.H} N={w.N} chunk={chunk} dtype={w.dtype} rope={rope} "
          f"carried={carried} out_grad={out_grad}", flush=True)
    x = generate(w, seed=seed, names=("q", "k", "v", "dout"))
    q, k, v, do = (to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v", "dout"))
    ang = oracle.rope3d_angles(*w.grid) if rope else None
    r = rope_for(w) if rope else None
    S_in = z_in = dS_out = dz_out = None
    dev_kw = {}
    if carried:
        S_in, z_in = _state_like(w, 1234)
        dev_kw.update(kv_in=torch.from_numpy(S_in).to(device()), ksum_in=torch.from_numpy(z_in).to(device()))
    if out_grad:
        rng = np.random.default_rng(4321)
        dS_out = (rng.standard_normal((w.B, w.H, 32, 32)) * 1e-3).astype(np.float32)
        dz_out = (rng.standard_normal((w.B, w.H, 32)) * 1e-4).astype(np.float32)
        dev_kw.update(dkv_out=torch.from_numpy(dS_out).to(device()), dksum_out=torch.from_numpy(dz_out).to(device()))
    dkv_in = torch.empty(w.B, w.H, 32, 32, device=device())
    dz_in = torch.empty(w.B, w.H, 32, device=device())
    dq, dk, dv = la.sana_linattn_backward(q, k, v, do, chunk=chunk, eps=w.eps, rope=r, dkv_in=dkv_in,
                                          dksum_in=dz_in, **dev_kw)
    f = x.f64
    ref = oracle.backward(f["q"], f["k"], f["v"], f["dout"], w.eps, angles=ang, chunk=chunk,
                          S_in=S_in, z_in=z_in, dS_out=dS_out, dz_out=dz_out)
    for got, want, name in zip((dq, dk, dv), ref[:3], ("dq", "dk", "dv")):
        check(to_np(got), want, w.dtype, f"{label} {name}")
    tol = 1e-5 if w.dtype == "f32" else 1e-4
    for got, want, name in ((dkv_in, ref[3], "dkv_in"), (dz_in, ref[4], "dksum_in")):
        err = rel_l2(to_np(got), want)
        print(f"{label} {name}: rel-L2 {err:.3e}", flush=True)
        assert err <= tol, f"{label} {name}: rel-L2 {err:.3e} > {tol}"
    return dq, dk, dv, dkv_in, dz_in


SMALL = [
    # (dtype, B, H, N, chunk, rope grid or None, carried, out_grad)
    ("f32", 1, 1, 2, None, None, False, False),
    ("f32", 1, 2, 33, None, None, False, False),
    ("f32", 2, 3, 257, None, None, True, True),
    ("f32", 1, 2, 100, 40, None, False, False),
    ("f32", 1, 2, 997, 128, None, True, True),
    ("f32", 1, 2, 120, 7, (2, 6, 10), True, True),
    ("f32", 1, 3, 1000, None, (4, 10, 25), False, False),
    ("bf16", 1, 1, 15, None, None, False, False),
    ("bf16", 2, 2, 1000, None, None, False, False),
    ("bf16", 1, 4, 5000, 4680, None, True, True),
    ("bf16", 1, 3, 2000, 333, (5, 20, 20), True, True),
    ("bf16", 1, 2, 4097, None, (17, 1, 241), False, False),
    # 14 chunks x 6 splits: 84 partials per head, so both finalize directions
    # walk two batches with chunk ends inside each
    ("bf16", 1, 2, 20000, 1500, None, True, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-B{c[1]}H{c[2]}N{c[3]}-L{c[4]}-rope{c[5] is not None}")
def test_backward_small(case):
    dtype, B, H, N, chunk, grid, carried, out_grad = case
    w = Workload(name="bwd_small", B=B, H=H, N=N, dtype=dtype, scale=0.5 if dtype == "bf16" else 1.0,
                 mode="rope" if grid else "noncausal", grid=grid)
    _run(w, chunk, rope=grid is not None, carried=carried, out_grad=out_grad, label="small")


@pytest.mark.parametrize("dtype,chunk", [("bf16", None), ("bf16", 300), ("f32", None), ("f32", 300)])
def test_backward_eps_zero_ragged(dtype, chunk):
    """eps = 0 with token ranges that end inside a 32-token tile: the rows
    padded past a range's end hold zeros, and their 1 / (den + eps) must not
    reach dS or dz (every real row has den > 0 here)."""
    w = Workload(name="bwd_eps0", B=1, H=3, N=1000, dtype=dtype, scale=0.5 if dtype == "bf16" else 1.0, eps=0.0)
    dq, dk, dv, dkv, dz = _run(w, chunk, label="eps0")
    for t in (dq, dk, dv, dkv, dz):
        assert bool(torch_mod().isfinite(t).all())


@pytest.mark.parametrize("name", ["sana16b_4096px", "video720p_rope3d", "video480p_blockcausal"])
def test_backward_full_size(name):
    w = WORKLOADS[name]
    chunk = w.chunk if w.mode == "block" else None
    _run(w, chunk, rope=w.mode == "rope", label=name)


def test_backward_single_token():
    """N = 1: O = V s / (s + eps) with s = phi(Q).phi(K), so dQ and dK are
    eps-sized: dphi(Q) = phi(K) (dO.(V - O)) / den and V - O = V eps / den.  In
    the kernels these are differences of two terms of size |phi(K)| |V.dO| /
    den (resp. |phi(Q)| ...), which cancel below fp32 resolution, so dQ and dK
    are held to an absolute bound of fp32 rounding on those terms; dV is O(1)
    and checked as usual."""
    w = Workload(name="bwd_one", B=2, H=3, N=1, dtype="f32", scale=1.0)
    x = generate(w, names=("q", "k", "v", "dout"))
    q, k, v, do = (to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v", "dout"))
    dq, dk, dv = la.sana_linattn_backward(q, k, v, do, eps=w.eps)
    f = x.f64
    ref = oracle.backward(f["q"], f["k"], f["v"], f["dout"], w.eps)
    check(to_np(dv), ref[2], "f32", "N=1 dv")
    phiq, phik = np.maximum(f["q"], 0.0), np.maximum(f["k"], 0.0)
    den = (phiq * phik).sum(-1, keepdims=True) + w.eps
    vdo = np.abs((f["v"] * f["dout"]).sum(-1, keepdims=True))
    for got, want, other, name in ((dq, ref[0], phik, "dq"), (dk, ref[1], phiq, "dk")):
        bound = 1e-5 * (other * vdo / den).max()
        err = np.abs(to_np(got) - want).max()
        print(f"N=1 {name}: max |diff| {err:.3e} (bound {bound:.3e})", flush=True)
        assert err <= bound, name


def test_backward_chunk_by_chunk_equals_whole_sequence():
    """The backward of a per-chunk block_forward loop, run chunk by chunk in
    reverse order passing dkv_in on as the previous chunk's dkv_out, matches the
    whole-sequence backward."""
    torch = torch_mod()
    w = reduced(WORKLOADS["video480p_blockcausal"], H=6, N=4 * 700, chunk=700)
    x = generate(w, names=("q", "k", "v", "dout"))
    q, k, v, do = (to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v", "dout"))
    dq, dk, dv = la.sana_linattn_backward(q, k, v, do, chunk=w.chunk, eps=w.eps)
    # forward states before each chunk
    kv = torch.zeros(w.B, w.H, 32, 32, device=device())
    z = torch.zeros(w.B, w.H, 32, device=device())
    starts = []
    for kc, vc in zip(split_chunks(k, w.chunk), split_chunks(v, w.chunk)):
        starts.append((kv.clone(), z.clone()))
        la.sana_linattn_state_update(kc, vc, kv, z)
    g_kv = torch.zeros(w.B, w.H, 32, 32, device=device())
    g_z = torch.zeros(w.B, w.H, 32, device=device())
    parts = {"dq": [], "dk": [], "dv": []}
    chunks = list(zip(split_chunks(q, w.chunk), split_chunks(k, w.chunk), split_chunks(v, w.chunk),
                      split_chunks(do, w.chunk)))
    for c in range(len(chunks) - 1, -1, -1):
        qc, kc, vc, dc = chunks[c]
        a, b, cc = la.sana_linattn_backward(qc, kc, vc, dc, eps=w.eps, kv_in=starts[c][0], ksum_in=starts[c][1],
                                            dkv_out=g_kv, dksum_out=g_z, dkv_in=g_kv, dksum_in=g_z)
        parts["dq"].insert(0, a)
        parts["dk"].insert(0, b)
        parts["dv"].insert(0, cc)
    for name, whole in (("dq", dq), ("dk", dk), ("dv", dv)):
        err = rel_l2(to_np(torch.cat(parts[name], dim=2)), to_np(whole))
        print(f"chunk-by-chunk vs whole sequence {name}: rel-L2 {err:.3e}", flush=True)
        assert err <= 2e-3, name


def test_backward_deterministic():
    w = reduced(WORKLOADS["sana06b_1024px"], H=8)
    x = generate(w, names=("q", "k", "v", "dout"))
    q, k, v, do = (to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v", "dout"))
    a = la.sana_linattn_backward(q, k, v, do, eps=w.eps)
    b = la.sana_linattn_backward(q, k, v, do, eps=w.eps)
    for s, t in zip(a, b):
        assert bool((s.view(torch_mod().int16) == t.view(torch_mod().int16)).all())


def test_backward_zero_rows_and_empty():
    """Rows with phi(Q) = 0 get dQ = 0 on their negative features and
    z dden on none (dden = 0 as num = 0); all-negative keys get dK = 0; N = 0
    writes nothing."""
    torch = torch_mod()
    w = reduced(WORKLOADS["sana06b_1024px"], B=1, H=2, N=300)
    x = generate(w, names=("q", "k", "v", "dout"))
    q, k, v, do = (to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v", "dout"))
    q[:, :, 5] = -torch.abs(q[:, :, 5])
    k[:, :, 7] = -torch.abs(k[:, :, 7])
    dq, dk, dv = la.sana_linattn_backward(q, k, v, do, eps=w.eps)
    assert bool((dq[:, :, 5] == 0).all()) and bool((dk[:, :, 7] == 0).all())
    empty = q[:, :, :0].contiguous()
    outs = la.sana_linattn_backward(empty, empty, empty, empty, eps=w.eps)
    assert all(t.numel() == 0 for t in outs)


@pytest.mark.parametrize("rope", [False, True])
def test_state_update_backward(rope):
    """dK, dV of <dkv, S> + dksum . z alone (the key pass) against the oracle's
    backward with a zero output gradient and that state gradient."""
    torch = torch_mod()
    w = WORKLOADS["video720p_rope3d"] if rope else reduced(WORKLOADS["sana16b_4096px"], H=12, N=5000)
    print(f"case state_update_backward rope={rope}: H={w.H} N={w.N}", flush=True)
    x = generate(w)
    k, v = (to_dev(x.raw[n], w.dtype) for n in ("k", "v"))
    rng = np.random.default_rng(77)
    dS = rng.standard_normal((w.B, w.H, 32, 32)).astype(np.float32)
    dz = rng.standard_normal((w.B, w.H, 32)).astype(np.float32)
    dk, dv = la.sana_linattn_state_update_backward(k, v, torch.from_numpy(dS).to(device()),
                                                   torch.from_numpy(dz).to(device()),
                                                   rope=rope_for(w) if rope else None)
    f = x.f64
    ang = oracle.rope3d_angles(*w.grid) if rope else None
    ref = oracle.backward(f["q"], f["k"], f["v"], np.zeros_like(f["q"]), w.eps, angles=ang, dS_out=dS, dz_out=dz)
    check(to_np(dk), ref[1], w.dtype, "state_update_backward dk")
    check(to_np(dv), ref[2], w.dtype, "state_update_backward dv")


# --------------------------------------------------------------------------
# backward from the forward's saved chunk states
# --------------------------------------------------------------------------

@pytest.mark.parametrize("label,base,changes,chunk,rope,carried,packed", [
    ("non-causal", "sana16b_4096px", dict(H=4, N=3000), None, False, False, False),
    ("block-causal, carried state", "video480p_blockcausal", dict(H=3, N=2000, chunk=500), 500, False, True, False),
    ("single chunk, carried state", "video480p_blockcausal", dict(H=3, N=900, chunk=900), 900, False, True, False),
    ("per-axis RoPE", "video720p_rope3d", dict(H=2, N=3 * 8 * 20, grid=(3, 8, 20)), 160, True, False, False),
    ("fp32", "noncausal_f32_b1h1n256", dict(H=3, N=700), 300, False, False, False),
    ("packed", "sana16b_4096px", dict(H=6, N=1000), None, False, False, True),
])
def test_backward_saved_equals_recompute(label, base, changes, chunk, rope, carried, packed):
    """sana_linattn_backward_saved, given the workspace of the forward call
    (forward, block_forward or block_causal), skips the state recompute and
    must give the recomputing backward's gradients bit for bit."""
    torch = torch_mod()
    w = reduced(WORKLOADS[base], **changes)
    print(f"case backward_saved {label}: H={w.H} N={w.N} chunk={chunk} dtype={w.dtype}", flush=True)
    x = generate(w, names=("q", "k", "v", "dout"))
    q, k, v, do = (to_dev(x.raw[n], w.dtype) for n in ("q", "k", "v", "dout"))
    if packed:
        buf = torch.empty(w.B, w.N, 4, w.H, w.D, dtype=q.dtype, device=device())
        for i, t in enumerate((q, k, v, do)):
            buf[:, :, i] = t.permute(0, 2, 1, 3)
        q, k, v, do = (buf[:, :, i].permute(0, 2, 1, 3) for i in range(4))
    r = la.rope3d_axes_device(*w.grid, device()) if rope else None
    kw = {}
    if carried:
        S_in, z_in = _state_like(w, 77)
        kw = dict(kv_in=torch.from_numpy(S_in).to(device()), ksum_in=torch.from_numpy(z_in).to(device()))
    L = w.N if chunk is None else chunk
    dt = la.SANA_DT_BF16 if w.dtype == "bf16" else la.SANA_DT_F32
    ws = torch.empty(max(la.backward_workspace_bytes(w.B, w.H, w.N, L, dtype=dt, has_rope=rope), 256),
                     dtype=torch.uint8, device=device())
    g = torch.Generator().manual_seed(3)
    dkv_out = (torch.randn(w.B, w.H, 32, 32, generator=g) * 1e-3).to(device())
    dz_out = (torch.randn(w.B, w.H, 32, generator=g) * 1e-4).to(device())
    if chunk is None:
        la.sana_linattn_forward(q, k, v, eps=w.eps, rope=r, workspace=ws)
    elif chunk >= w.N:
        la.sana_linattn_block_forward(q, k, v, eps=w.eps, rope=r, workspace=ws, **kw)
    else:
        la.sana_linattn_block_causal(q, k, v, chunk, eps=w.eps, rope=r, workspace=ws, **kw)
    outs = []
    for saved in (True, False):
        dkv_in = torch.empty(w.B, w.H, 32, 32, device=device())
        dz_in = torch.empty(w.B, w.H, 32, device=device())
        common = dict(chunk=chunk, dkv_out=dkv_out, dksum_out=dz_out, dkv_in=dkv_in, dksum_in=dz_in, eps=w.eps, rope=r)
        if saved:
            grads = la.sana_linattn_backward_saved(q, k, v, do, ws, **common)
        else:
            grads = la.sana_linattn_backward(q, k, v, do, **common, **kw)
        outs.append(tuple(grads) + (dkv_in, dz_in))
    for a, b, name in zip(outs[0], outs[1], ("dq", "dk", "dv", "dkv_in", "dksum_in")):
        assert torch.equal(a, b), f"{label}: {name} differs from the recomputing backward"
