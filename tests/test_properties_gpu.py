"""Property test (Hypothesis) of the HIP path against the float64 oracle over
random shapes: batch, heads, ragged token counts (1 .. 2600, so one to several
split partials and a ragged last tile), the three forms (non-causal, 3D RoPE in
either table form, block-causal at a random chunk length) and both I/O dtypes,
each held to the tolerance of its dtype (rel-L2 <= 1e-5 for fp32; rel-L2 <=
4e-3 and floored max rel <= 2e-2 for bf16)."""

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import linear_attention_diffusion_amd as la
import oracle
from gpu_util import device, inputs_on_device, to_np
from metrics import check
from workloads import WORKLOADS, generate, reduced

pytestmark = pytest.mark.gpu


@st.composite
def cases(draw):
    mode = draw(st.sampled_from(["noncausal", "block", "rope"]))
    dtype = draw(st.sampled_from(["bf16", "bf16", "f32"]))
    B = draw(st.integers(1, 2))
    H = draw(st.integers(1, 5))
    grid, chunk = None, None
    if mode == "rope":
        grid = (draw(st.integers(1, 3)), draw(st.integers(1, 12)), draw(st.integers(1, 40)))
        N = grid[0] * grid[1] * grid[2]
    else:
        N = draw(st.integers(1, 2600))
        if mode == "block":
            chunk = draw(st.integers(1, N))
    seed = draw(st.integers(0, 2**31 - 1))
    form = draw(st.sampled_from(["table", "axes"]))
    base = WORKLOADS["noncausal_f32_b1h1n256"] if dtype == "f32" else WORKLOADS["sana16b_4096px"]
    w = reduced(base, B=B, H=H, N=N, mode=mode, grid=grid, chunk=chunk, seed=seed)
    return w, form


@settings(max_examples=30, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(case=cases())
def test_hip_path_matches_the_oracle(case):
    w, form = case
    x = generate(w)
    q, k, v = inputs_on_device(x)
    f = x.f64
    tag = f"B={w.B} H={w.H} N={w.N} {w.mode} {w.dtype} chunk={w.chunk} grid={w.grid} seed={w.seed}"
    if w.mode == "rope":
        rope = (la.rope3d_axes_device if form == "axes" else la.rope3d_device)(*w.grid, device())
        o = la.sana_linattn_forward(q, k, v, eps=w.eps, rope=rope)
        ref = oracle.linattn(f["q"], f["k"], f["v"], w.eps, angles=oracle.rope3d_angles(*w.grid))
    elif w.mode == "block":
        o = la.sana_linattn_block_causal(q, k, v, w.chunk, eps=w.eps)
        ref, _, _ = oracle.block_causal(f["q"], f["k"], f["v"], w.chunk, w.eps)
    else:
        o = la.sana_linattn_forward(q, k, v, eps=w.eps)
        ref = oracle.linattn(f["q"], f["k"], f["v"], w.eps)
    check(to_np(o), ref, w.dtype, tag)
