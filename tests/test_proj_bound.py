"""CPU checks of the element-wise bound used for the fused projection's GPU
parity (proj_bound.py): the oracle's own result passes it, and results with a
plausible kernel mistake planted in them (computed here from the oracle's
pieces on the CPU) fail it."""

import numpy as np
import pytest

import oracle
from proj_bound import check_projected_apply, check_projected_state, oracle_weights
from workloads import PROJECTIONS, generate_projection, reduced


@pytest.fixture(scope="module")
def case():
    x = generate_projection(reduced(PROJECTIONS["sana16b_4096px_kv_proj"], B=2, N=600, C=96, H=3, seed=21))
    wk, wv = oracle_weights(x.f64["w_k"], 3), oracle_weights(x.f64["w_v"], 3)
    return x, wk, wv


def _state(k, v):
    return oracle.kv_state(k, v)


def _proj(x, w, rounded=True):
    y = np.matmul(x.f64["x"][:, None], w[None])
    return oracle.round_bf16(y) if rounded else y


def test_oracle_result_passes(case):
    x, wk, wv = case
    S, z = oracle.projected_kv_state(x.f64["x"], wk, wv)
    ok, report = check_projected_state(S, z, x)
    assert ok, report
    ok, report = check_projected_state(S, z, x, any_order=True)
    assert ok, report


def test_fp32_rounding_of_the_projection_passes(case):
    """K and V summed in float32 (any order numpy picks), then rounded: what a
    correct kernel may produce."""
    x, wk, wv = case
    x32 = x.f64["x"].astype(np.float32)[:, None]
    k = oracle.round_bf16(np.matmul(x32, wk.astype(np.float32)[None]).astype(np.float64))
    v = oracle.round_bf16(np.matmul(x32, wv.astype(np.float32)[None]).astype(np.float64))
    S, z = _state(k, v)
    ok, report = check_projected_state(S, z, x, any_order=True)
    assert ok, report


@pytest.mark.parametrize("mistake", ["unrounded", "dropped_token", "transposed", "relu_on_v", "z_without_relu",
                                     "swapped_heads", "truncated"])
def test_planted_mistakes_fail(case, mistake):
    x, wk, wv = case
    k, v = _proj(x, wk), _proj(x, wv)
    if mistake == "unrounded":
        S, z = _state(_proj(x, wk, False), _proj(x, wv, False))
    elif mistake == "dropped_token":
        S, z = _state(k[:, :, :-1], v[:, :, :-1])
    elif mistake == "transposed":
        S, z = _state(k, v)
        S = np.swapaxes(S, -1, -2)
    elif mistake == "relu_on_v":
        S, z = _state(k, np.maximum(v, 0.0))
    elif mistake == "z_without_relu":
        S, _ = _state(k, v)
        z = k.sum(axis=-2)
    elif mistake == "swapped_heads":
        S, z = _state(k[:, ::-1], v[:, ::-1])
    elif mistake == "truncated":
        # bf16 by dropping the low half of the float32 bits instead of rounding
        def trunc(y):
            u = y.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
            return u.view(np.float32).astype(np.float64)
        S, z = _state(trunc(_proj(x, wk, False)), trunc(_proj(x, wv, False)))
    ok, report = check_projected_state(S, z, x)
    assert not ok, f"{mistake} passed the bound: {report}"


@pytest.fixture(scope="module")
def rope_case():
    grid = (2, 5, 7)
    x = generate_projection(reduced(PROJECTIONS["sana16b_4096px_kv_proj"], B=2, N=60, C=64, H=2, seed=22))
    wk, wv = oracle_weights(x.f64["w_k"], 2), oracle_weights(x.f64["w_v"], 2)
    return x, wk, wv, oracle.rope3d_angles(*grid)


def _rotated_state(x, wk, wv, angles, off, rotate):
    k, v = _proj(x, wk), _proj(x, wv)
    phik = np.maximum(k, 0.0)
    S = np.matmul(np.swapaxes(rotate(phik, angles[off:off + x.workload.N]), -1, -2), v)
    return S, phik.sum(axis=-2)


def test_rope_oracle_and_float32_rotation_pass(rope_case):
    x, wk, wv, angles = rope_case
    S, z = oracle.projected_kv_state(x.f64["x"], wk, wv, angles, 10)
    ok, report = check_projected_state(S, z, x, angles=angles, pos_offset=10)
    assert ok, report

    def rot32(y, a):
        # float32 cos/sin and float32 products, as the kernel computes them
        c, s = np.cos(a).astype(np.float32), np.sin(a).astype(np.float32)
        y = y.astype(np.float32)
        out = np.empty_like(y)
        out[..., 0::2] = y[..., 0::2] * c - y[..., 1::2] * s
        out[..., 1::2] = y[..., 0::2] * s + y[..., 1::2] * c
        return out.astype(np.float64)

    S32, z32 = _rotated_state(x, wk, wv, angles, 10, rot32)
    ok, report = check_projected_state(S32, z32, x, angles=angles, pos_offset=10)
    assert ok, report


@pytest.mark.parametrize("mistake", ["unrotated", "sign", "offset", "rotated_z"])
def test_rope_planted_mistakes_fail(rope_case, mistake):
    x, wk, wv, angles = rope_case
    if mistake == "unrotated":
        S, z = oracle.projected_kv_state(x.f64["x"], wk, wv)
    elif mistake == "sign":
        S, z = oracle.projected_kv_state(x.f64["x"], wk, wv, -angles, 10)
    elif mistake == "offset":
        S, z = oracle.projected_kv_state(x.f64["x"], wk, wv, angles, 0)
    else:
        S, _ = oracle.projected_kv_state(x.f64["x"], wk, wv, angles, 10)
        phik = np.maximum(_proj(x, wk), 0.0)
        z = oracle.rotate_pairs(phik, angles[10:10 + x.workload.N]).sum(axis=-2)
    ok, report = check_projected_state(S, z, x, angles=angles, pos_offset=10)
    assert not ok, f"{mistake} passed the bound: {report}"


# ---------------------------------------------------------------------------
# the bound for the query projection fused with the apply step
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def apply_case():
    p = reduced(PROJECTIONS["sana16b_4096px_kv_proj"], B=2, N=700, C=96, H=3, seed=22)
    x = generate_projection(p, names=("x", "w_q"))
    rng = np.random.default_rng(5)
    k = oracle.round_bf16(rng.standard_normal((2, 3, 900, 32)))
    v = oracle.round_bf16(rng.standard_normal((2, 3, 900, 32)))
    S, z = oracle.kv_state(k, v)
    return x, oracle_weights(x.f64["w_q"], 3), S, z


def _out(q, S, z, eps=1e-6, angles=None, offset=0):
    return oracle.round_bf16(oracle.apply_state(q, S, z, eps, angles, offset))


def test_apply_oracle_result_passes(apply_case):
    x, wq, S, z = apply_case
    ok, report = check_projected_apply(_out(_proj(x, wq), S, z), x, S, z, 1e-6)
    assert ok, report


def test_apply_float32_query_and_flipped_roundings_pass(apply_case):
    """Q summed in float32 then rounded, and Q with every feature that sits
    next to a rounding boundary moved to its other neighbour: outputs a correct
    kernel may produce."""
    x, wq, S, z = apply_case
    x32 = x.f64["x"].astype(np.float32)[:, None]
    q32 = oracle.round_bf16(np.matmul(x32, wq.astype(np.float32)[None]).astype(np.float64))
    ok, report = check_projected_apply(_out(q32, S, z), x, S, z, 1e-6, any_order=True)
    assert ok, report
    exact = _proj(x, wq, False)
    q = oracle.round_bf16(exact)
    delta = 2.0 * (96 / 32 + 32) * 2.0 ** -24 * np.matmul(np.abs(x.f64["x"])[:, None], np.abs(wq)[None])
    lo, hi = oracle.round_bf16(exact - delta), oracle.round_bf16(exact + delta)
    flipped = np.where(lo != q, lo, hi)
    assert np.count_nonzero(flipped != q) > 0
    ok, report = check_projected_apply(_out(flipped, S, z), x, S, z, 1e-6)
    assert ok, report


@pytest.mark.parametrize("mistake", ["unrounded", "truncated", "num_without_relu", "den_without_relu",
                                     "swapped_heads", "state_transposed", "last_token_dropped"])
def test_apply_planted_mistakes_fail(apply_case, mistake):
    x, wq, S, z = apply_case
    q = _proj(x, wq)
    if mistake == "unrounded":
        o = _out(_proj(x, wq, False), S, z)
    elif mistake == "truncated":
        u = _proj(x, wq, False).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
        o = _out(u.view(np.float32).astype(np.float64), S, z)
    elif mistake == "num_without_relu":
        o = np.matmul(q, S) / (np.matmul(np.maximum(q, 0.0), z[..., :, None]) + 1e-6)
    elif mistake == "den_without_relu":
        o = np.matmul(np.maximum(q, 0.0), S) / (np.matmul(q, z[..., :, None]) + 1e-6)
    elif mistake == "swapped_heads":
        o = _out(q, S[:, ::-1], z[:, ::-1])
    elif mistake == "state_transposed":
        o = _out(q, np.swapaxes(S, -1, -2), z)
    elif mistake == "last_token_dropped":
        o = _out(q, S, z)
        o[:, :, -1] = 0.0
    ok, report = check_projected_apply(o, x, S, z, 1e-6)
    assert not ok, f"{mistake} passed the bound: {report}"


@pytest.mark.parametrize("mistake", [None, "rotation_dropped", "positions_from_zero", "rotated_denominator"])
def test_apply_rope_bound(apply_case, mistake):
    x, wq, S, z = apply_case
    ang = oracle.rope3d_angles(4, 10, 20)
    q = _proj(x, wq)
    if mistake is None:
        o = _out(q, S, z, angles=ang, offset=30)
    elif mistake == "rotation_dropped":
        o = _out(q, S, z)
    elif mistake == "positions_from_zero":
        o = _out(q, S, z, angles=ang, offset=0)
    else:
        p = oracle.rotate_pairs(np.maximum(q, 0.0), ang[30:30 + q.shape[-2]])
        o = np.matmul(p, S) / (np.matmul(p, z[..., :, None]) + 1e-6)
    ok, report = check_projected_apply(o, x, S, z, 1e-6, angles=ang, pos_offset=30)
    assert ok == (mistake is None), f"{mistake}: {report}"
