"""CPU checks of the element-wise bound used for the fused projection's GPU
parity (proj_bound.py): the oracle's own result passes it, and results with a
plausible kernel mistake planted in them (computed here from the oracle's
pieces on the CPU) fail it."""

import numpy as np
import pytest

import oracle
from proj_bound import check_projected_state, oracle_weights
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
