"""Property tests (Hypothesis) of the fused projections against the float64
oracle over random shapes: batch 1-2, 1-12 heads (so partial head groups on
both sides; 13-20 in the large class), C = 32, 64 or 96 channels (one to
three channel steps, so the RoPE angle table lands in each of the three LDS
stages), token counts in three classes up to 14000 (one block, ragged last
blocks, up to a few hundred tiles: halves and quarters only, or whole tiles
with split tails),
and 3D RoPE in either table form at a random position offset into a random
latent grid.  Each example runs sana_linattn_project_state from a zero state
and sana_linattn_project_apply against an independent state that the oracle
builds from other random keys and values, both held to the element-wise bounds
derived in proj_bound.py."""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, to_dev, to_np, torch_mod
from proj_bound import check_projected_apply, check_projected_state
from workloads import PROJECTIONS, generate_projection, reduced

pytestmark = pytest.mark.gpu

FULL = PROJECTIONS["sana16b_4096px_kv_proj"]


@st.composite
def proj_cases(draw):
    # size classes, drawn first so that every run reaches the large grids
    # (above 256 tiles on both sides: whole tiles, then split tails)
    size = draw(st.sampled_from(["small", "medium", "large"]))
    B = draw(st.integers(1, 2))
    H = draw(st.integers(13, 20) if size == "large" else st.integers(1, 12))
    C = draw(st.sampled_from([32, 64, 96]))
    form = draw(st.sampled_from([None, "axes", "table"]))
    lo, hi = {"small": (1, 600), "medium": (600, 4000), "large": (9000, 14000)}[size]
    grid, offset = None, 0
    if form is None:
        N = draw(st.integers(lo, hi))
    else:
        # a latent grid within T <= 6, H_l <= 32, W_l <= 80 (per-axis tables of
        # at most 6*4 + 32*6 + 80*6 = 696 entries); the large class takes
        # grids of at least 5 x 28 x 64 = 8960 positions
        if size == "large":
            grid = (draw(st.integers(5, 6)), draw(st.integers(28, 32)), draw(st.integers(64, 80)))
        else:
            grid = (draw(st.integers(1, 6)), draw(st.integers(1, 32)), draw(st.integers(1, 80)))
        total = grid[0] * grid[1] * grid[2]
        N = draw(st.integers(min(lo, total), min(hi, total)))
        offset = draw(st.integers(0, total - N))
    seed = draw(st.integers(0, 2**31 - 1))
    return B, N, C, H, form, grid, offset, seed


def _independent_state(B, H, seed):
    """An fp32 state for the apply from the oracle: S, z of 1024 other random
    bf16 keys and values per head (unit variance)."""
    rng = np.random.default_rng(seed)
    k = oracle.round_bf16(rng.standard_normal((B, H, 1024, 32)))
    v = oracle.round_bf16(rng.standard_normal((B, H, 1024, 32)))
    S, z = oracle.kv_state(k, v)
    return S.astype(np.float32), z.astype(np.float32)


@settings(max_examples=16, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(case=proj_cases())
def test_fused_projections_match_the_oracle(case):
    B, N, C, H, form, grid, offset, seed = case
    torch = torch_mod()
    print(f"case B={B} N={N} C={C} H={H} rope={form} grid={grid} offset={offset} seed={seed}", flush=True)
    x = generate_projection(reduced(FULL, B=B, N=N, C=C, H=H, seed=seed), names=("x", "w_k", "w_v", "w_q"))
    rope, angles = None, None
    if form is not None:
        rope = (la.rope3d_axes_device if form == "axes" else la.rope3d_device)(*grid, device()).at(offset)
        angles = oracle.rope3d_angles(*grid)
    xs, wk, wv, wq = (to_dev(x.raw[n], "bf16") for n in ("x", "w_k", "w_v", "w_q"))

    kv = torch.zeros(B, H, 32, 32, device=device())
    z = torch.zeros(B, H, 32, device=device())
    la.sana_linattn_project_state(xs, wk, wv, kv, z, rope=rope)
    ok, report = check_projected_state(to_np(kv), to_np(z), x, angles=angles, pos_offset=offset)
    assert ok, "project_state: " + report

    S, zs = _independent_state(B, H, seed + 1)
    o = la.sana_linattn_project_apply(xs, wq, torch.from_numpy(S).to(device()), torch.from_numpy(zs).to(device()),
                                      eps=1e-6, rope=rope)
    ok, report = check_projected_apply(to_np(o), x, S, zs, 1e-6, angles=angles, pos_offset=offset)
    assert ok, "project_apply: " + report
