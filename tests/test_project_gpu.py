"""GPU parity of sana_linattn_project_state: the key/value projection fused with
the state update, against the float64 oracle's projected_kv_state (K = x W_k^T,
V = x W_v^T rounded to bf16, then S = sum phi(K)^T V, z = sum phi(K)).

The tolerance is the element-wise bound derived in proj_bound.py."""

import numpy as np
import pytest

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, to_dev, to_np, torch_mod
from metrics import BF16_REL_L2, rel_l2
from proj_bound import check_projected_apply, check_projected_state, oracle_weights
from workloads import PROJECTIONS, generate_projection, reduced

pytestmark = pytest.mark.gpu

FULL = PROJECTIONS["sana16b_4096px_kv_proj"]


def _check_state(*args, **kw):
    ok, report = check_projected_state(*args, **kw)
    print(report, flush=True)
    assert ok, report


def _run(x, kv=None, z=None, rope=None):
    torch = torch_mod()
    p = x.workload
    dev = device()
    xs, wk, wv = (to_dev(x.raw[n], "bf16") for n in ("x", "w_k", "w_v"))
    if kv is None:
        kv = torch.zeros(p.B, p.H, 32, 32, device=dev)
        z = torch.zeros(p.B, p.H, 32, device=dev)
    la.sana_linattn_project_state(xs, wk, wv, kv, z, rope=rope)
    return kv, z


# (B, N, C, H): one 256-token block; ragged tails with an odd head count (the
# last group of four heads is partial); several ranges (partials + finalize);
# more than 128 blocks, so each range spans two blocks; a single head; three
# head groups of four, the last with one head, over two batches.  The grid
# deals each XCD a run of tiles and cuts the tiles of the run's last round
# (count % 32 of them) into parts when that helps: four one-head quarters when
# at most 8, two two-head halves when at most 16.  Runs here: up to 9 tiles
# (quarters only), except 65 tiles (runs of 8 and 9: quarters and halves);
# 272 and 264 tiles (runs of 34 and 33: whole tiles, then quarters; the second
# with a ragged block and three heads in the last group); 132 tiles of
# two-block ranges (runs of 17, whole tiles only, and 16, halves only).
CASES = [(1, 256, 32, 2), (2, 700, 96, 3), (1, 1000, 64, 4), (1, 5000, 128, 5), (1, 33000, 32, 2), (1, 300, 64, 1),
         (2, 600, 64, 9), (2, 17408, 32, 6), (2, 16740, 32, 7), (1, 33700, 32, 7)]


@pytest.mark.parametrize("B,N,C,H", CASES)
def test_project_state_matches_oracle(B, N, C, H):
    print(f"case project_state B={B} N={N} C={C} H={H}", flush=True)
    x = generate_projection(reduced(FULL, B=B, N=N, C=C, H=H, seed=N + C))
    kv, z = _run(x)
    _check_state(to_np(kv), to_np(z), x)


def test_project_state_max_channels():
    """C = 65536, the largest channel count the call accepts (2048 channel
    steps; x rows of 128 KB)."""
    print("case project_state C=65536", flush=True)
    x = generate_projection(reduced(FULL, B=1, N=300, C=65536, H=3, seed=41))
    kv, z = _run(x)
    _check_state(to_np(kv), to_np(z), x)


def test_project_state_accumulates_in_place():
    """The call adds to the states it is given, as state_update does."""
    torch = torch_mod()
    x = generate_projection(reduced(FULL, B=1, N=1200, C=64, H=3, seed=5))
    g = torch.Generator().manual_seed(3)
    kv0 = torch.randn(1, 3, 32, 32, generator=g)
    z0 = torch.rand(1, 3, 32, generator=g) * 100
    print("case project_state in place", flush=True)
    kv, z = _run(x, kv0.to(device()), z0.to(device()))
    _check_state(to_np(kv), to_np(z), x, kv0=kv0.double().numpy(), z0=z0.double().numpy())


def test_project_state_empty_leaves_state():
    torch = torch_mod()
    x = generate_projection(reduced(FULL, B=1, N=0, C=64, H=2))
    kv0 = torch.full((1, 2, 32, 32), 1.5, device=device())
    z0 = torch.full((1, 2, 32), 2.5, device=device())
    print("case project_state N=0", flush=True)
    kv, z = _run(x, kv0.clone(), z0.clone())
    assert bool((kv == kv0).all()) and bool((z == z0).all())


def test_project_state_equals_two_pass_path():
    """Against the unfused path: a bf16 torch projection writes K and V, then
    sana_linattn_state_update reads them.  The two roundings of K and V can
    differ only where the fp32 sums fall on opposite sides of a bf16 boundary:
    both results must lie within the oracle's bound."""
    torch = torch_mod()
    p = reduced(FULL, B=2, N=3000, C=256, H=6, seed=11)
    x = generate_projection(p)
    print("case project_state vs two-pass", flush=True)
    kv, z = _run(x)
    xs, wk, wv = (to_dev(x.raw[n], "bf16") for n in ("x", "w_k", "w_v"))
    x2 = xs.reshape(p.B * p.N, p.C)
    k = (x2 @ wk.t().contiguous()).reshape(p.B, p.N, p.H, 32).permute(0, 2, 1, 3).contiguous()
    v = (x2 @ wv.t().contiguous()).reshape(p.B, p.N, p.H, 32).permute(0, 2, 1, 3).contiguous()
    kv2 = torch.zeros_like(kv)
    z2 = torch.zeros_like(z)
    la.sana_linattn_state_update(k, v, kv2, z2)
    _check_state(to_np(kv), to_np(z), x)
    _check_state(to_np(kv2), to_np(z2), x, any_order=True)


def test_full_4096px_layer_sampled_heads():
    """The Sana-1.6B 4096 px key/value projection (16384 tokens, C = 2240, 70
    heads) in the launch configuration the benchmark times; the oracle computes
    five of the heads, including both heads of the first and last pair."""
    x = generate_projection(FULL)
    print("case project_state full 4096 px", flush=True)
    kv, z = _run(x)
    heads = [0, 1, 37, 68, 69]
    _check_state(to_np(kv)[:, heads], to_np(z)[:, heads], x, heads)


def _same(a, b, what):
    torch = torch_mod()
    assert bool((a.view(torch.int32) == b.view(torch.int32)).all()), f"{what}: the two RoPE forms differ"


# the first three run as quarter tiles (one head each); the last, 96 tiles in
# runs of 12, as half tiles
@pytest.mark.parametrize("B,N,C,H,grid,offset", [(2, 480, 64, 3, (3, 8, 20), 0), (1, 300, 96, 2, (4, 10, 12), 150),
                                                 (1, 1000, 32, 5, (5, 10, 20), 0), (1, 12288, 32, 6, (12, 32, 32), 0)])
def test_project_state_rope(B, N, C, H, grid, offset):
    """Keys rotated by the 3D RoPE at positions offset .. offset + N - 1, with
    the full tables and with the per-axis tables (bit-identical to each
    other), against the oracle."""
    print(f"case project_state rope B={B} N={N} C={C} H={H} grid={grid} offset={offset}", flush=True)
    x = generate_projection(reduced(FULL, B=B, N=N, C=C, H=H, seed=N + 7))
    table = la.rope3d_device(*grid, device()).at(offset)
    axes = la.rope3d_axes_device(*grid, device()).at(offset)
    kv_t, z_t = _run(x, rope=table)
    kv_a, z_a = _run(x, rope=axes)
    _same(kv_a, kv_t, "S")
    _same(z_a, z_t, "z")
    _check_state(to_np(kv_a), to_np(z_a), x, angles=oracle.rope3d_angles(*grid), pos_offset=offset)


def test_full_720p_layer_rope_sampled_heads():
    """The SANA-Video 720p layer's keys (21 x 22 x 40 = 18480 tokens, C = 2240,
    70 heads) with the per-axis 3D RoPE; the oracle computes four heads."""
    grid = (21, 22, 40)
    x = generate_projection(reduced(FULL, N=grid[0] * grid[1] * grid[2], seed=3))
    print("case project_state full 720p rope", flush=True)
    kv, z = _run(x, rope=la.rope3d_axes_device(*grid, device()))
    heads = [0, 1, 36, 69]
    _check_state(to_np(kv)[:, heads], to_np(z)[:, heads], x, heads, angles=oracle.rope3d_angles(*grid))


# ---------------------------------------------------------------------------
# query projection fused with the apply step
# ---------------------------------------------------------------------------

def _state_for(p, seed):
    """A realistic state for the apply: the oracle's state of another draw of
    K and V (unit variance, N tokens), rounded to fp32 (the values both sides
    use)."""
    rng = np.random.default_rng(seed)
    k = oracle.round_bf16(rng.standard_normal((p.B, p.H, p.N or 1, 32)))
    v = oracle.round_bf16(rng.standard_normal((p.B, p.H, p.N or 1, 32)))
    S, z = oracle.kv_state(k, v)
    return S.astype(np.float32), z.astype(np.float32)


def _run_apply(x, S, z, eps=1e-6, rope=None, o=None):
    torch = torch_mod()
    xs, wq = to_dev(x.raw["x"], "bf16"), to_dev(x.raw["w_q"], "bf16")
    return la.sana_linattn_project_apply(xs, wq, torch.from_numpy(S).to(device()), torch.from_numpy(z).to(device()),
                                         o=o, eps=eps, rope=rope)


def _check_apply(*args, **kw):
    ok, report = check_projected_apply(*args, **kw)
    print(report, flush=True)
    assert ok, report


# Tile kinds (see CASES above; here a whole tile is eight heads, a half four
# heads, a quarter four heads and 128 tokens): the first seven run as
# quarters; 272 tiles (runs of 34 per XCD) and 264 (runs of 33, a ragged last
# block, six heads in the second group) as whole tiles, then quarters; 96
# tiles (runs of 12, a ragged last block) as halves.
@pytest.mark.parametrize("B,N,C,H", [(1, 256, 32, 4), (2, 700, 96, 3), (1, 1000, 64, 6), (1, 5000, 128, 5),
                                     (1, 300, 64, 1), (2, 600, 64, 11), (1, 520, 32, 16), (2, 17408, 32, 12),
                                     (1, 33700, 32, 14), (1, 12132, 32, 12)])
def test_project_apply_matches_oracle(B, N, C, H):
    print(f"case project_apply B={B} N={N} C={C} H={H}", flush=True)
    x = generate_projection(reduced(FULL, B=B, N=N, C=C, H=H, seed=N + C + 1), names=("x", "w_q"))
    S, z = _state_for(x.workload, 7)
    o = _run_apply(x, S, z)
    _check_apply(to_np(o), x, S, z, 1e-6)


def test_project_apply_eps_zero_ragged():
    """eps = 0 with a ragged last block: the rows past N, whose queries read as
    zero (0 / 0), must not reach the output."""
    x = generate_projection(reduced(FULL, B=2, N=700, C=64, H=3, seed=31), names=("x", "w_q"))
    S, z = _state_for(x.workload, 12)
    print("case project_apply eps=0", flush=True)
    o = _run_apply(x, S, z, eps=0.0)
    _check_apply(to_np(o), x, S, z, 0.0)


def test_project_apply_max_channels():
    print("case project_apply C=65536", flush=True)
    x = generate_projection(reduced(FULL, B=1, N=300, C=65536, H=3, seed=42), names=("x", "w_q"))
    S, z = _state_for(x.workload, 13)
    _check_apply(to_np(_run_apply(x, S, z)), x, S, z, 1e-6)


def test_project_apply_empty_touches_nothing():
    torch = torch_mod()
    x = generate_projection(reduced(FULL, B=1, N=0, C=64, H=2), names=("x", "w_q"))
    S, z = _state_for(reduced(x.workload, N=100), 11)
    o = torch.full((1, 2, 0, 32), 1.0, dtype=torch.bfloat16, device=device())
    print("case project_apply N=0", flush=True)
    assert _run_apply(x, S, z, o=o) is o


@pytest.mark.parametrize("N", [25500, 25444])
def test_project_apply_many_blocks_ragged(N):
    """300 tiles (3 batch rows x 100 blocks x 1 group of eight heads, H = 6):
    more than one round of resident workgroups (one per CU), and every batch
    row ends in a ragged block (156 tokens, or 100, which leaves the block's
    second 128 tokens empty).  The last XCD's run ends with blocks 295 .. 299
    cut into quarter tiles of 128 tokens, so with N = 25444 one quarter of the
    last block holds no token at all."""
    print(f"case project_apply many blocks N={N}", flush=True)
    x = generate_projection(reduced(FULL, B=3, N=N, C=64, H=6, seed=N), names=("x", "w_q"))
    S, z = _state_for(reduced(x.workload, N=2000), 10)
    o = _run_apply(x, S, z)
    _check_apply(to_np(o), x, S, z, 1e-6)


# (grid, offset, N, C, H): C = 64, 96 and 32 give 2, 3 and 1 channel steps,
# so the angle table of the epilogue sits in each of the three LDS stages; the
# third case has two groups of eight heads (the second partial) and a ragged
# last block.  These run as quarter tiles; the last case (96 tiles in runs of
# 12) as half tiles.
@pytest.mark.parametrize("grid,offset,N,C,H", [((3, 8, 20), 0, 480, 64, 6), ((4, 10, 12), 150, 330, 64, 6),
                                               ((5, 10, 20), 0, 1000, 96, 9), ((4, 10, 12), 0, 480, 32, 3),
                                               ((12, 32, 32), 0, 12288, 32, 6)])
def test_project_apply_rope_and_strided_output(grid, offset, N, C, H):
    """Queries rotated by the 3D RoPE (both table forms, bit-identical), and
    outputs written straight into a [B, N, H, D] buffer."""
    torch = torch_mod()
    x = generate_projection(reduced(FULL, B=2, N=N, C=C, H=H, seed=17 + C), names=("x", "w_q"))
    S, z = _state_for(x.workload, 8)
    table = la.rope3d_device(*grid, device()).at(offset)
    axes = la.rope3d_axes_device(*grid, device()).at(offset)
    print(f"case project_apply rope grid={grid} offset={offset} N={N} C={C} H={H}", flush=True)
    o_t = _run_apply(x, S, z, rope=table)
    o_bnhd = torch.empty(2, N, H, 32, dtype=torch.bfloat16, device=device()).permute(0, 2, 1, 3)
    o_a = _run_apply(x, S, z, rope=axes, o=o_bnhd)
    assert bool((o_a.contiguous().view(torch.int16) == o_t.view(torch.int16)).all()), "forms or layouts differ"
    _check_apply(to_np(o_a), x, S, z, 1e-6, angles=oracle.rope3d_angles(*grid), pos_offset=offset)


def test_project_apply_full_720p_rope_sampled_heads():
    """The SANA-Video 720p layer's queries (21 x 22 x 40 = 18480 tokens,
    C = 2240, 70 heads) with the per-axis 3D RoPE, in the launch configuration
    the benchmark times; the oracle computes four heads, including the last,
    partial group of eight."""
    grid = (21, 22, 40)
    x = generate_projection(reduced(FULL, N=grid[0] * grid[1] * grid[2], seed=5), names=("x", "w_q"))
    S, z = _state_for(reduced(FULL, N=4096), 14)
    print("case project_apply full 720p rope", flush=True)
    o = _run_apply(x, S, z, rope=la.rope3d_axes_device(*grid, device()))
    heads = [0, 9, 42, 69]
    _check_apply(to_np(o)[:, heads], x, S, z, 1e-6, heads=heads, angles=oracle.rope3d_angles(*grid))


def test_project_apply_full_4096px_sampled_heads():
    """The Sana-1.6B 4096 px layer's queries (16384 tokens, C = 2240, 70 heads)
    in the launch configuration the benchmark times; the oracle computes five
    heads, including the last, partial group of eight (six heads)."""
    x = generate_projection(FULL, names=("x", "w_q"))
    S, z = _state_for(reduced(FULL, N=4096), 9)
    print("case project_apply full 4096 px", flush=True)
    o = _run_apply(x, S, z)
    heads = [0, 3, 35, 68, 69]
    _check_apply(to_np(o)[:, heads], x, S, z, 1e-6, heads=heads)


def test_projected_layer_end_to_end():
    """project_state then project_apply: the whole attention of a layer from
    its input x.  The state is checked within its bound, the output within the
    apply's bound given that state, and both the fused and the unfused path
    (torch GEMMs + forward) against the oracle's attention of the
    bf16-rounded projections by rel-L2."""
    torch = torch_mod()
    p = reduced(FULL, B=2, N=1500, C=128, H=4, seed=23)
    x = generate_projection(p, names=("x", "w_k", "w_v", "w_q"))
    print("case projected layer end to end", flush=True)
    xs, wk, wv, wq = (to_dev(x.raw[n], "bf16") for n in ("x", "w_k", "w_v", "w_q"))
    kv = torch.zeros(p.B, p.H, 32, 32, device=device())
    z = torch.zeros(p.B, p.H, 32, device=device())
    la.sana_linattn_project_state(xs, wk, wv, kv, z)
    o = la.sana_linattn_project_apply(xs, wq, kv, z)
    _check_state(to_np(kv), to_np(z), x)
    _check_apply(to_np(o), x, to_np(kv), to_np(z), 1e-6)
    f = x.f64
    proj = [oracle.round_bf16(np.matmul(f["x"][:, None], oracle_weights(f[n], p.H)[None]))
            for n in ("w_q", "w_k", "w_v")]
    want = oracle.linattn(*proj, 1e-6)
    x2 = xs.reshape(p.B * p.N, p.C)
    q, k, v = ((x2 @ w.t().contiguous()).reshape(p.B, p.N, p.H, 32).permute(0, 2, 1, 3).contiguous()
               for w in (wq, wk, wv))
    unfused = la.sana_linattn_forward(q, k, v)
    for name, got in (("fused", o), ("unfused", unfused)):
        l2 = rel_l2(to_np(got), want)
        print(f"{name} layer: rel-L2 {l2:.3e} against the oracle", flush=True)
        assert l2 <= BF16_REL_L2, name
