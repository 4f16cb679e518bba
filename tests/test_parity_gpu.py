"""GPU parity: the HIP path, called through the C ABI, against the float64
oracle on the same seeded inputs, element by element.

Full-size cases run every workload at its real shape in the launch
configuration the benchmark times; the smaller cases span several tiles with
ragged tails.  bf16: rel-L2 <= 4e-3 and floored max rel err <= 2e-2; fp32:
rel-L2 <= 1e-5 (see tests/metrics.py)."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import (device, inputs_on_device, rope_for, run_block_chunks, run_forward, to_dev, to_np,
                      torch_mod)
from metrics import check, rel_l2
from workloads import WORKLOADS, f64_from_bf16_bits, generate, reduced

pytestmark = pytest.mark.gpu


def _oracle_for(x, angles=None):
    w = x.workload
    f = x.f64
    if w.mode == "block":
        return oracle.block_causal(f["q"], f["k"], f["v"], w.chunk, w.eps, angles=angles)[0]
    return oracle.linattn(f["q"], f["k"], f["v"], w.eps, angles=angles)


# --------------------------------------------------------------------------
# the five workloads at full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_workload(name):
    w = WORKLOADS[name]
    print(f"case {name}: B={w.B} H={w.H} N={w.N} mode={w.mode} dtype={w.dtype}", flush=True)
    x = generate(w)
    angles = oracle.rope3d_angles(*w.grid) if w.mode == "rope" else None
    if w.mode == "block":
        o, kv, z = run_block_chunks(x, w.chunk)
        ref, S_ref, z_ref = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], w.chunk, w.eps)
        assert rel_l2(kv, S_ref) <= 1e-5 and rel_l2(z, z_ref) <= 1e-6
    else:
        o = run_forward(x, rope=rope_for(w) if w.mode == "rope" else None)
        ref = _oracle_for(x, angles)
    check(o, ref, w.dtype, name)


# --------------------------------------------------------------------------
# ragged and small shapes, every mode and dtype
# --------------------------------------------------------------------------

SMALL = [
    # (dtype, mode, B, H, N, chunk, grid)
    ("bf16", "noncausal", 1, 1, 1, None, None),
    ("bf16", "noncausal", 1, 3, 15, None, None),
    ("bf16", "noncausal", 2, 2, 33, None, None),
    ("bf16", "noncausal", 1, 5, 257, None, None),
    ("bf16", "noncausal", 3, 4, 1000, None, None),
    ("bf16", "noncausal", 1, 2, 4097, None, None),
    ("bf16", "noncausal", 8, 40, 7, None, None),
    ("bf16", "noncausal", 1, 1, 70001, None, None),
    ("f32", "noncausal", 1, 1, 1, None, None),
    ("f32", "noncausal", 2, 3, 100, None, None),
    ("f32", "noncausal", 1, 2, 3001, None, None),
    ("bf16", "rope", 1, 2, 1 * 3 * 5, None, (1, 3, 5)),
    ("bf16", "rope", 2, 3, 4 * 7 * 9, None, (4, 7, 9)),
    ("bf16", "rope", 1, 2, 5 * 22 * 40, None, (5, 22, 40)),
    ("f32", "rope", 1, 2, 3 * 6 * 7, None, (3, 6, 7)),
    ("bf16", "block", 1, 2, 100, 40, None),
    ("bf16", "block", 2, 3, 997, 128, None),
    ("bf16", "block", 1, 2, 5 * 333, 333, None),
    ("f32", "block", 1, 2, 300, 64, None),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}N{c[4]}")
def test_small_and_ragged(case):
    dtype, mode, B, H, N, chunk, grid = case
    base = WORKLOADS["noncausal_f32_b1h1n256"] if dtype == "f32" else WORKLOADS["sana16b_4096px"]
    w = reduced(base, B=B, H=H, N=N, mode=mode, chunk=chunk, grid=grid, seed=N)
    print(f"case {w}", flush=True)
    x = generate(w)
    angles = oracle.rope3d_angles(*grid) if mode == "rope" else None
    if mode == "block":
        o, _, _ = run_block_chunks(x, chunk)
    else:
        o = run_forward(x, rope=rope_for(w) if mode == "rope" else None)
    check(o, _oracle_for(x, angles), dtype, str(case))


def test_block_causal_with_rope():
    """Block mode with RoPE reads the table at global positions (pos_offset)."""
    grid = (6, 10, 12)
    w = reduced(WORKLOADS["video480p_blockcausal"], H=3, N=6 * 10 * 12, chunk=2 * 10 * 12, grid=grid)
    x = generate(w)
    angles = oracle.rope3d_angles(*grid)
    o, _, _ = run_block_chunks(x, w.chunk, rope=rope_for(w))
    ref, _, _ = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], w.chunk, w.eps, angles=angles)
    check(o, ref, "bf16", "block-causal RoPE")


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_empty_is_noop():
    torch = torch_mod()
    e = torch.empty(1, 2, 0, 32, dtype=torch.bfloat16, device=device())
    o = la.sana_linattn_forward(e, e, e)
    assert o.shape == e.shape
    kv = torch.ones(1, 2, 32, 32, device=device())
    z = torch.ones(1, 2, 32, device=device())
    la.sana_linattn_state_update(e, e, kv, z)
    torch.cuda.synchronize()
    assert torch.all(kv == 1) and torch.all(z == 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_zero_rows(dtype):
    """All-negative keys, or all-negative queries, give exact zeros (0 / eps)."""
    torch = torch_mod()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 3, 300, 32, generator=g).to(tdt).to(device())
    k_neg = (-torch.rand(1, 3, 300, 32, generator=g) - 0.1).to(tdt).to(device())
    v = torch.randn(1, 3, 300, 32, generator=g).to(tdt).to(device())
    o = la.sana_linattn_forward(q, k_neg, v)
    assert torch.all(o == 0)
    o = la.sana_linattn_forward(-q.abs() - 0.1, v, q)
    assert torch.all(o == 0)


def test_constant_v_gives_the_constant():
    """Non-RoPE: V = c gives O_i = c s_i / (s_i + eps); rounded to bf16 this is c."""
    torch = torch_mod()
    w = reduced(WORKLOADS["sana16b_4096px"], H=4, N=5000)
    x = generate(w)
    q, k, _ = inputs_on_device(x)
    c = torch.randn(32).to(torch.bfloat16)
    v = c.to(device()).expand(1, 4, 5000, 32).contiguous()
    o = la.sana_linattn_forward(q, k, v)
    pos = (torch.clamp(q.float(), min=0).sum(-1) > 0)   # rows with some positive query feature
    want = c.to(device()).expand_as(o)
    assert torch.equal(o[pos], want[pos])
    assert torch.all(o[~pos] == 0)


def test_small_workspace_is_rejected():
    torch = torch_mod()
    w = reduced(WORKLOADS["sana16b_4096px"], H=2, N=512)
    q, k, v = inputs_on_device(generate(w))
    ws = torch.empty(64, dtype=torch.uint8, device=device())
    with pytest.raises(la.SanaError) as e:
        la.sana_linattn_forward(q, k, v, workspace=ws)
    assert e.value.code == la.SANA_ERR_WORKSPACE


# --------------------------------------------------------------------------
# invariants on the device
# --------------------------------------------------------------------------

def test_deterministic():
    w = reduced(WORKLOADS["sana16b_4096px"], H=6, N=9000)
    x = generate(w)
    assert np.array_equal(run_forward(x), run_forward(x))


def test_identity_rope_is_bit_identical_to_plain():
    torch = torch_mod()
    w = reduced(WORKLOADS["sana16b_4096px"], H=3, N=2000)
    x = generate(w)
    ident = la.Rope(torch.ones(2000, 16, device=device()), torch.zeros(2000, 16, device=device()))
    assert np.array_equal(run_forward(x, rope=ident), run_forward(x))
    xf = generate(reduced(WORKLOADS["noncausal_f32_b1h1n256"], H=2, N=2000))
    assert np.array_equal(run_forward(xf, rope=ident), run_forward(xf))


def test_single_chunk_equals_forward():
    w = reduced(WORKLOADS["sana16b_4096px"], H=3, N=3000)
    x = generate(w)
    o_block, _, _ = run_block_chunks(x, 3000)
    assert np.array_equal(o_block, run_forward(x))


def test_read_only_chunk_matches_commit_and_leaves_state():
    torch = torch_mod()
    w = reduced(WORKLOADS["video480p_blockcausal"], H=3, N=1200, chunk=600)
    x = generate(w)
    q, k, v = inputs_on_device(x)
    kv = torch.zeros(1, 3, 32, 32, device=device())
    z = torch.zeros(1, 3, 32, device=device())
    first = [t[:, :, :600].contiguous() for t in (q, k, v)]
    second = [t[:, :, 600:].contiguous() for t in (q, k, v)]
    la.sana_linattn_block_forward(*first, kv_in=kv, ksum_in=z, kv_out=kv, ksum_out=z)
    kv_saved, z_saved = kv.clone(), z.clone()
    o_ro = la.sana_linattn_block_forward(*second, kv_in=kv, ksum_in=z)      # denoising step: read only
    torch.cuda.synchronize()
    assert torch.equal(kv, kv_saved) and torch.equal(z, z_saved)
    o_commit = la.sana_linattn_block_forward(*second, kv_in=kv, ksum_in=z, kv_out=kv, ksum_out=z)
    assert torch.equal(o_ro, o_commit)
    ref, S_ref, z_ref = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], 600, w.eps)
    check(to_np(o_commit), ref[:, :, 600:], "bf16", "read-only / commit chunk")
    assert rel_l2(to_np(kv), S_ref) <= 1e-5


def test_save_restore_and_causality():
    """Copying the state to the host and back mid-sequence changes nothing, and
    changing a later chunk leaves earlier outputs bit-identical."""
    torch = torch_mod()
    w = reduced(WORKLOADS["video480p_blockcausal"], H=4, N=4 * 500, chunk=500)
    x = generate(w)
    o_ref, kv_ref, z_ref = run_block_chunks(x, 500)
    q, k, v = inputs_on_device(x)
    kv = torch.zeros(1, 4, 32, 32, device=device())
    z = torch.zeros(1, 4, 32, device=device())
    outs = []
    for c in range(4):
        sl = slice(500 * c, 500 * (c + 1))
        if c == 2:
            kv = torch.from_numpy(kv.cpu().numpy().copy()).to(device())
            z = torch.from_numpy(z.cpu().numpy().copy()).to(device())
        outs.append(la.sana_linattn_block_forward(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                                                  v[:, :, sl].contiguous(), kv_in=kv, ksum_in=z,
                                                  kv_out=kv, ksum_out=z))
    assert np.array_equal(to_np(torch.cat(outs, dim=2)), o_ref)
    # perturb chunks 2 and 3
    x2 = generate(w)
    rng = np.random.default_rng(99)
    for n in ("q", "k", "v"):
        x2.raw[n][:, :, 1000:] = x2.raw[n][:, :, 1000:][..., rng.permutation(32)]
    o2, _, _ = run_block_chunks(x2, 500)
    assert np.array_equal(o2[:, :, :1000], o_ref[:, :, :1000])
    assert not np.array_equal(o2[:, :, 1000:], o_ref[:, :, 1000:])


def test_state_update_in_pieces():
    torch = torch_mod()
    w = reduced(WORKLOADS["sana16b_4096px"], H=3, N=6000)
    x = generate(w)
    _, k, v = inputs_on_device(x)
    kv = torch.zeros(1, 3, 32, 32, device=device())
    z = torch.zeros(1, 3, 32, device=device())
    la.sana_linattn_state_update(k[:, :, :2500].contiguous(), v[:, :, :2500].contiguous(), kv, z)
    la.sana_linattn_state_update(k[:, :, 2500:].contiguous(), v[:, :, 2500:].contiguous(), kv, z)
    S_ref, z_ref = oracle.kv_state(x.f64["k"], x.f64["v"])
    assert rel_l2(to_np(kv), S_ref) <= 1e-5
    assert rel_l2(to_np(z), z_ref) <= 1e-6
    kv1 = torch.zeros_like(kv)
    z1 = torch.zeros_like(z)
    la.sana_linattn_state_update(k, v, kv1, z1)
    assert rel_l2(to_np(kv1), to_np(kv)) <= 1e-6


def test_state_update_with_rope_and_offset():
    torch = torch_mod()
    grid = (4, 10, 12)
    w = reduced(WORKLOADS["video720p_rope3d"], H=2, N=480, grid=grid)
    x = generate(w)
    _, k, v = inputs_on_device(x)
    rope = rope_for(w)
    kv = torch.zeros(1, 2, 32, 32, device=device())
    z = torch.zeros(1, 2, 32, device=device())
    la.sana_linattn_state_update(k[:, :, :200].contiguous(), v[:, :, :200].contiguous(), kv, z, rope=rope.at(0))
    la.sana_linattn_state_update(k[:, :, 200:].contiguous(), v[:, :, 200:].contiguous(), kv, z, rope=rope.at(200))
    S_ref, z_ref = oracle.kv_state(x.f64["k"], x.f64["v"], angles=oracle.rope3d_angles(*grid))
    assert rel_l2(to_np(kv), S_ref) <= 1e-5
    assert rel_l2(to_np(z), z_ref) <= 1e-6


def test_apply_matches_forward_and_oracle():
    """forward == state_update into a zero state followed by apply (same
    kernels, same order of sums), and apply on its own matches the oracle's
    apply_state for a given state."""
    torch = torch_mod()
    for rope_grid in (None, (3, 10, 20)):
        N = 3000 if rope_grid is None else 3 * 10 * 20
        w = reduced(WORKLOADS["sana16b_4096px"], H=5, N=N, seed=11)
        x = generate(w)
        q, k, v = inputs_on_device(x)
        rope = None if rope_grid is None else la.rope3d_device(*rope_grid, device())
        kv = torch.zeros(1, 5, 32, 32, device=device())
        z = torch.zeros(1, 5, 32, device=device())
        la.sana_linattn_state_update(k, v, kv, z, rope=rope)
        o_apply = la.sana_linattn_apply(q, kv, z, eps=w.eps, rope=rope)
        o_fwd = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=rope)
        assert torch.equal(o_apply, o_fwd)
        angles = None if rope_grid is None else oracle.rope3d_angles(*rope_grid)
        ref = oracle.apply_state(x.f64["q"], to_np(kv), to_np(z), w.eps, angles=angles)
        check(to_np(o_apply), ref, "bf16", f"apply on a given state (rope={rope_grid})")


@pytest.mark.parametrize("H,N,grid", [(1, 4096, None), (1, 8192, None), (70, 4680, None), (3, 700, (7, 10, 10)),
                                       (2, 2000, (5, 20, 20))])
def test_block_forward_matches_state_update_then_apply(H, N, grid):
    """From the same non-zero carried state, block_forward's in-place commit
    and outputs equal bit for bit those of state_update followed by apply
    (the same sums in the same order), for 1 to 32 partial states per head; a
    read-only call gives the same outputs."""
    torch = torch_mod()
    w = reduced(WORKLOADS["video720p_rope3d"] if grid else WORKLOADS["sana16b_4096px"], H=H, N=N, grid=grid,
                seed=23)
    print(f"case block_forward vs state_update + apply H={H} N={N} grid={grid}", flush=True)
    x = generate(w)
    q, k, v = inputs_on_device(x)
    rope = rope_for(w) if grid else None
    g = torch.Generator().manual_seed(5)
    kv0 = (torch.rand(1, H, 32, 32, generator=g) * 10).to(device())
    z0 = (torch.rand(1, H, 32, generator=g) * 10).to(device())
    kv_a, z_a = kv0.clone(), z0.clone()
    la.sana_linattn_state_update(k, v, kv_a, z_a, rope=rope)
    o_a = la.sana_linattn_apply(q, kv_a, z_a, eps=w.eps, rope=rope)
    o_ro = la.sana_linattn_block_forward(q, k, v, kv_in=kv0, ksum_in=z0, eps=w.eps, rope=rope)
    kv_b, z_b = kv0.clone(), z0.clone()
    o_b = la.sana_linattn_block_forward(q, k, v, kv_in=kv_b, ksum_in=z_b, kv_out=kv_b, ksum_out=z_b, eps=w.eps,
                                        rope=rope)
    torch.cuda.synchronize()
    assert torch.equal(kv_b, kv_a) and torch.equal(z_b, z_a)
    assert torch.equal(o_b, o_a) and torch.equal(o_ro, o_a)
    ang = oracle.rope3d_angles(*grid) if grid else None
    S_ref, z_ref = oracle.kv_state(x.f64["k"], x.f64["v"], angles=ang)
    assert rel_l2(to_np(kv_b), S_ref + to_np(kv0).astype(np.float64)) <= 1e-5
    assert rel_l2(to_np(z_b), z_ref + to_np(z0).astype(np.float64)) <= 1e-6


# --------------------------------------------------------------------------
# whole-sequence block-causal call
# --------------------------------------------------------------------------

def _run_sequence(x, chunk, rope=None, with_state=False, S0=None, z0=None):
    torch = torch_mod()
    w = x.workload
    q, k, v = inputs_on_device(x)
    kv = z = None
    if with_state:
        kv = torch.from_numpy(S0.astype(np.float32)).to(device())
        z = torch.from_numpy(z0.astype(np.float32)).to(device())
    o = la.sana_linattn_block_causal(q, k, v, chunk, kv_in=kv, ksum_in=z, kv_out=kv, ksum_out=z, eps=w.eps,
                                     rope=rope)
    return to_np(o), (None if kv is None else to_np(kv)), (None if z is None else to_np(z))


def test_block_causal_sequence_full_size():
    w = WORKLOADS["video480p_blockcausal"]
    x = generate(w)
    o, _, _ = _run_sequence(x, w.chunk)
    ref, _, _ = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], w.chunk, w.eps)
    check(o, ref, "bf16", "block-causal sequence call, 10 x 4680")


@pytest.mark.parametrize("N,chunk,dtype", [(100, 40, "bf16"), (997, 128, "bf16"), (5000, 4680, "bf16"),
                                           (4680, 4680, "bf16"), (64, 1, "bf16"), (2000, 333, "f32"),
                                           (20000, 1500, "bf16")])
def test_block_causal_sequence_cases(N, chunk, dtype):
    base = WORKLOADS["noncausal_f32_b1h1n256"] if dtype == "f32" else WORKLOADS["video480p_blockcausal"]
    w = reduced(base, B=2, H=3, N=N, mode="block", chunk=chunk, seed=N + chunk)
    x = generate(w)
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((2, 3, 32, 32))
    z0 = np.abs(rng.standard_normal((2, 3, 32))) * 50
    o, S, z = _run_sequence(x, chunk, with_state=True, S0=S0, z0=z0)
    # the oracle from the same carried state
    Sr, zr = S0.astype(np.float32).astype(np.float64), z0.astype(np.float32).astype(np.float64)
    ref = np.empty(x.f64["q"].shape)
    for s0 in range(0, N, chunk):
        sl = slice(s0, min(N, s0 + chunk))
        ref[:, :, sl], Sr, zr = oracle.block_forward(x.f64["q"][:, :, sl], x.f64["k"][:, :, sl],
                                                     x.f64["v"][:, :, sl], Sr, zr, w.eps)
    check(o, ref, dtype, f"block-causal sequence N={N} chunk={chunk} with carried state")
    assert rel_l2(S, Sr) <= 1e-5 and rel_l2(z, zr) <= 1e-6


def test_block_causal_sequence_rope_and_chunk_loop_agree():
    grid = (6, 10, 12)
    w = reduced(WORKLOADS["video480p_blockcausal"], H=3, N=6 * 10 * 12, chunk=2 * 10 * 12, grid=grid)
    x = generate(w)
    rope = rope_for(w)
    o_seq, _, _ = _run_sequence(x, w.chunk, rope=rope)
    o_loop, _, _ = run_block_chunks(x, w.chunk, rope=rope)
    ref, _, _ = oracle.block_causal(x.f64["q"], x.f64["k"], x.f64["v"], w.chunk, w.eps,
                                    angles=oracle.rope3d_angles(*grid))
    check(o_seq, ref, "bf16", "block-causal sequence with RoPE")
    assert rel_l2(o_seq, o_loop) <= 4e-3
    # one chunk covering everything is the plain forward
    o_one, _, _ = _run_sequence(x, 10 ** 6)
    assert np.array_equal(o_one, run_forward(x))


# --------------------------------------------------------------------------
# geometry extremes: one very long head (the split cap: 64 partials per head),
# and many short heads (one workgroup per head, no finalize)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,N", [(1, 1, 1 << 20), (64, 64, 64), (2, 3, 300001)])
def test_geometry_extremes(B, H, N):
    w = reduced(WORKLOADS["sana16b_4096px"], B=B, H=H, N=N)
    print(f"case extremes: B={B} H={H} N={N}", flush=True)
    x = generate(w)
    o = run_forward(x)
    check(o, oracle.linattn(x.f64["q"], x.f64["k"], x.f64["v"], w.eps), "bf16", f"extremes B{B}H{H}N{N}")


def test_tensors_beyond_2gib():
    """Each of Q, K, V, O spans 2.24 GB (70 heads x 500000 tokens, bf16), so
    head 67 straddles byte offset 2^31 and heads 68, 69 lie beyond it.
    Sampled heads, including those, are checked against the oracle run on that
    head alone (the oracle cannot take the whole tensor in seconds)."""
    torch = torch_mod()
    w = reduced(WORKLOADS["sana16b_4096px"], H=70, N=500_000)
    assert (w.H - 1) * w.N * w.D * 2 > 2 ** 31
    print("case tensors beyond 2 GiB: B=1 H=70 N=500000", flush=True)
    x = generate(w, with_f64=False)
    q, k, v = inputs_on_device(x)
    o = la.sana_linattn_forward(q, k, v, eps=w.eps)
    torch.cuda.synchronize()
    del q, k, v
    for h in (0, 35, 67, 69):
        head = [f64_from_bf16_bits(x.raw[n][:, h:h + 1]) for n in ("q", "k", "v")]
        check(to_np(o[:, h:h + 1]), oracle.linattn(*head, w.eps), "bf16", f"head {h} of a 2.24 GB tensor")
