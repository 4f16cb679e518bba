"""Property tests (Hypothesis) of the float64 oracle over random small shapes,
seeds, chunkings and RoPE grids: the structural facts the pages state, checked
at shapes the fixed pins do not reach.

- Linear form = quadratic form ("SANA-Video" news article, "Design details":
  splitting along the tokens is mathematically the full pairwise form; "Sana"
  research note, Model architecture item 2): shared terms computed once).
- Block-causal: chunked recurrence = masked quadratic form; the final state is
  the full sequence's state; a later chunk never changes an earlier one's
  outputs ("SANA-Video" paper notes 2.3; news article "Design details").
- RoPE after the ReLU and in the numerator only ("SANA-Video" paper notes 2.2):
  identity angles reduce to the plain form; denominators ignore the angles;
  a common shift of every position leaves the outputs unchanged.
- Linearity in V, positive rescaling of Q (eps = 0), joint permutation of
  (K, V) in the non-causal form.
"""

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


def _qkv(seed, B, H, N, D, scale=0.5):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, H, N, D)) * scale for _ in range(3))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


shapes = st.tuples(st.integers(1, 2), st.integers(1, 3), st.integers(1, 40), st.sampled_from([1, 2, 4, 8, 32]))


@SETTINGS
@given(shape=shapes, seed=st.integers(0, 2**31 - 1))
def test_linear_equals_quadratic(shape, seed):
    q, k, v = _qkv(seed, *shape)
    assert _rel(oracle.linattn(q, k, v, 1e-6), oracle.brute_force(q, k, v, 1e-6)) < 1e-10


@SETTINGS
@given(shape=shapes, chunk=st.integers(1, 45), seed=st.integers(0, 2**31 - 1))
def test_block_causal_equals_masked_quadratic(shape, chunk, seed):
    q, k, v = _qkv(seed, *shape)
    o, S, z = oracle.block_causal(q, k, v, chunk, 1e-6)
    assert _rel(o, oracle.brute_force(q, k, v, 1e-6, chunk=chunk)) < 1e-10
    S_all, z_all = oracle.kv_state(k, v)
    assert _rel(S, S_all) < 1e-12 and _rel(z, z_all) < 1e-12


@SETTINGS
@given(shape=shapes, chunk=st.integers(1, 20), cut=st.integers(1, 39), seed=st.integers(0, 2**31 - 1))
def test_later_chunks_never_change_earlier_outputs(shape, chunk, cut, seed):
    B, H, N, D = shape
    q, k, v = _qkv(seed, *shape)
    c_end = ((min(cut, N - 1) // chunk) + 1) * chunk  # first token after the chunk holding `cut`
    if c_end >= N:
        return
    o1, _, _ = oracle.block_causal(q, k, v, chunk, 1e-6)
    rng = np.random.default_rng(seed + 1)
    q2, k2, v2 = (x.copy() for x in (q, k, v))
    for x in (q2, k2, v2):
        x[..., c_end:, :] = rng.standard_normal(x[..., c_end:, :].shape)
    o2, _, _ = oracle.block_causal(q2, k2, v2, chunk, 1e-6)
    assert np.array_equal(o1[..., :c_end, :], o2[..., :c_end, :])


grids = st.tuples(st.integers(1, 3), st.integers(1, 4), st.integers(1, 5))


@SETTINGS
@given(grid=grids, H=st.integers(1, 2), chunk=st.one_of(st.none(), st.integers(1, 30)),
       seed=st.integers(0, 2**31 - 1))
def test_rope_forms(grid, H, chunk, seed):
    N = grid[0] * grid[1] * grid[2]
    q, k, v = _qkv(seed, 1, H, N, 32)
    angles = oracle.rope3d_angles(*grid)
    if chunk is None:
        o = oracle.linattn(q, k, v, 1e-6, angles=angles)
    else:
        o, _, _ = oracle.block_causal(q, k, v, chunk, 1e-6, angles=angles)
    assert _rel(o, oracle.brute_force(q, k, v, 1e-6, angles=angles, chunk=chunk)) < 1e-10
    # identity angles: the plain form
    zero = np.zeros_like(angles)
    assert _rel(oracle.linattn(q, k, v, 1e-6, angles=zero), oracle.linattn(q, k, v, 1e-6)) < 1e-12
    # the key sum (and so the denominator) ignores the angles
    S, z = oracle.kv_state(k, v, angles)
    S0, z0 = oracle.kv_state(k, v)
    assert np.array_equal(z, z0)


@SETTINGS
@given(grid=grids, shift=st.integers(1, 50), seed=st.integers(0, 2**31 - 1))
def test_rope_common_shift(grid, shift, seed):
    """R_{i+d}^T R_{j+d} = R_i^T R_j: shifting every position along one axis by
    the same amount leaves the outputs unchanged."""
    T, Hl, Wl = grid
    N = T * Hl * Wl
    q, k, v = _qkv(seed, 1, 1, N, 32)
    a = oracle.rope3d_angles(T, Hl, Wl)
    big = oracle.rope3d_angles(T + shift, Hl, Wl)
    b = big[shift * Hl * Wl: shift * Hl * Wl + N]          # every t moved by `shift`
    assert _rel(oracle.linattn(q, k, v, 1e-6, angles=b), oracle.linattn(q, k, v, 1e-6, angles=a)) < 1e-9


@SETTINGS
@given(shape=shapes, a=st.floats(-3, 3), b=st.floats(-3, 3), seed=st.integers(0, 2**31 - 1))
def test_linearity_in_v(shape, a, b, seed):
    q, k, v = _qkv(seed, *shape)
    v2 = np.random.default_rng(seed + 7).standard_normal(v.shape)
    lhs = oracle.linattn(q, k, a * v + b * v2, 1e-6)
    rhs = a * oracle.linattn(q, k, v, 1e-6) + b * oracle.linattn(q, k, v2, 1e-6)
    assert np.max(np.abs(lhs - rhs)) <= 1e-9 * (1 + np.max(np.abs(rhs)))


@SETTINGS
@given(shape=shapes, s=st.floats(0.01, 100), seed=st.integers(0, 2**31 - 1))
def test_query_scale_invariance_without_eps(shape, s, seed):
    q, k, v = _qkv(seed, *shape)
    phiq = np.maximum(q, 0)
    den = phiq @ np.maximum(k, 0).sum(axis=-2)[..., :, None]
    keep = den[..., 0] > 0                                      # eps = 0: rows with a zero denominator are 0/0
    with np.errstate(invalid="ignore"):
        o1 = oracle.linattn(q, k, v, 0.0)[keep]
        o2 = oracle.linattn(s * q, k, v, 0.0)[keep]
    assert np.max(np.abs(o1 - o2), initial=0.0) <= 1e-11 * (1 + np.max(np.abs(o1), initial=0.0))


@SETTINGS
@given(shape=shapes, seed=st.integers(0, 2**31 - 1))
def test_joint_key_value_permutation(shape, seed):
    q, k, v = _qkv(seed, *shape)
    perm = np.random.default_rng(seed + 3).permutation(k.shape[-2])
    assert _rel(oracle.linattn(q, k[..., perm, :], v[..., perm, :], 1e-6), oracle.linattn(q, k, v, 1e-6)) < 1e-12


@pytest.mark.parametrize("D", [1, 32])
def test_zero_queries_give_zero(D):
    """phi(Q_i) = 0 gives exactly 0 / eps = 0 (a fixed case beside the random ones)."""
    q, k, v = _qkv(5, 1, 2, 9, D)
    q[..., 3, :] = -np.abs(q[..., 3, :])
    o = oracle.linattn(q, k, v, 1e-6)
    assert np.array_equal(o[..., 3, :], np.zeros_like(o[..., 3, :]))
