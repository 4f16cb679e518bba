"""Pins for the float64 oracle: each pin checks the oracle against something other
than itself (exact rational brute force, closed forms, invariants the pages'
statements imply).  Every pin takes the oracle implementation as an argument so
that the mutation tests can run the same pins against deliberately broken
copies of the oracle and show that each planted mistake is caught.
"""

import numpy as np

from exact_ref import exact_attention, exact_gradients, exact_state, token_causal_recurrence

EPS = 1e-6


def _dyadic(rng, shape, lo=-2.0, hi=2.0):
    """Small dyadic values (multiples of 1/4): exact in bf16, fp32 and float64."""
    return np.round(rng.uniform(lo, hi, size=shape) * 4.0) / 4.0


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / scale if a.size else 0.0
    assert err <= rtol, f"{what}: max |diff|/max|ref| = {err:.3e} > {rtol:.1e}"


# --------------------------------------------------------------------------
# Exact brute force (quadratic definition, rational arithmetic)
# --------------------------------------------------------------------------

def pin_exact_noncausal(impl):
    rng = np.random.default_rng(11)
    for N, D in [(1, 1), (2, 2), (3, 4), (5, 4), (6, 2)]:
        q, k, v = (_dyadic(rng, (N, D)) for _ in range(3))
        want = exact_attention(q, k, v, EPS)
        got = impl.linattn(q[None, None], k[None, None], v[None, None], EPS)[0, 0]
        _close(got, want, 1e-12, f"linear vs exact quadratic N={N} D={D}")
        got_bf = impl.brute_force(q[None, None], k[None, None], v[None, None], EPS)[0, 0]
        _close(got_bf, want, 1e-12, f"numpy quadratic vs exact N={N} D={D}")


def pin_exact_state(impl):
    rng = np.random.default_rng(12)
    k, v = _dyadic(rng, (7, 4)), _dyadic(rng, (7, 4))
    S_want, z_want = exact_state(k, v)
    S, z = impl.kv_state(k[None, None], v[None, None])
    _close(S[0, 0], S_want, 0.0, "S = relu(K)^T V (row d = key feature, column e = value feature)")
    _close(z[0, 0], z_want, 0.0, "z = sum relu(K_j)")


def pin_exact_rope(impl):
    rng = np.random.default_rng(13)
    for N, D in [(2, 2), (4, 4), (5, 6)]:
        q, k, v = (_dyadic(rng, (N, D)) for _ in range(3))
        ang = rng.uniform(-3.0, 3.0, size=(N, D // 2))
        want = exact_attention(q, k, v, EPS, np.cos(ang), np.sin(ang))
        got = impl.linattn(q[None, None], k[None, None], v[None, None], EPS, angles=ang)[0, 0]
        _close(got, want, 1e-12, f"RoPE linear vs exact quadratic N={N} D={D}")
        got_bf = impl.brute_force(q[None, None], k[None, None], v[None, None], EPS, angles=ang)[0, 0]
        _close(got_bf, want, 1e-12, f"RoPE numpy quadratic vs exact N={N} D={D}")


def pin_exact_block(impl):
    rng = np.random.default_rng(14)
    for N, D, L in [(5, 2, 2), (6, 4, 3), (7, 4, 1), (4, 2, 4), (5, 2, 9)]:
        q, k, v = (_dyadic(rng, (N, D)) for _ in range(3))
        want = exact_attention(q, k, v, EPS, chunk=L)
        got, _, _ = impl.block_causal(q[None, None], k[None, None], v[None, None], L, EPS)
        _close(got[0, 0], want, 1e-12, f"chunked recurrence vs exact masked quadratic N={N} L={L}")
        got_bf = impl.brute_force(q[None, None], k[None, None], v[None, None], EPS, chunk=L)[0, 0]
        _close(got_bf, want, 1e-12, f"numpy masked quadratic vs exact N={N} L={L}")


def pin_exact_block_rope(impl):
    rng = np.random.default_rng(15)
    N, D, L = 6, 4, 4
    q, k, v = (_dyadic(rng, (N, D)) for _ in range(3))
    ang = rng.uniform(-3.0, 3.0, size=(N, D // 2))
    want = exact_attention(q, k, v, EPS, np.cos(ang), np.sin(ang), chunk=L)
    got, _, _ = impl.block_causal(q[None, None], k[None, None], v[None, None], L, EPS, angles=ang)
    _close(got[0, 0], want, 1e-12, "block-causal RoPE vs exact masked quadratic")


def pin_token_causal(impl):
    """Chunks of one token reduce to the inclusive token-causal recurrence."""
    rng = np.random.default_rng(16)
    q, k, v = (_dyadic(rng, (6, 4)) for _ in range(3))
    want = token_causal_recurrence(q, k, v, EPS)
    got, _, _ = impl.block_causal(q[None, None], k[None, None], v[None, None], 1, EPS)
    _close(got[0, 0], want, 1e-12, "chunk length 1 vs token-causal recurrence")


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def pin_closed_forms(impl):
    rng = np.random.default_rng(21)
    D = 32
    # N = 1: O = v * s / (s + eps), s = relu(q).relu(k)
    q, k, v = (rng.standard_normal((1, 1, 1, D)) for _ in range(3))
    s = np.sum(np.maximum(q, 0) * np.maximum(k, 0))
    _close(impl.linattn(q, k, v, EPS), v * s / (s + EPS), 1e-14, "N=1 closed form")
    # one-hot relu(Q_i) = e_a -> O_i = sum_j relu(K_ja) V_j / (sum_j relu(K_ja) + eps)
    N = 40
    k, v = rng.standard_normal((1, 1, N, D)), rng.standard_normal((1, 1, N, D))
    for a in (0, 7, 31):
        q = -np.ones((1, 1, 1, D))
        q[..., a] = 1.0
        w = np.maximum(k[0, 0, :, a], 0)
        want = (w @ v[0, 0]) / (w.sum() + EPS)
        _close(impl.apply_state(q, *impl.kv_state(k, v), EPS)[0, 0, 0], want, 1e-13,
               f"one-hot query on feature {a}")
    # all keys negative -> every output is exactly 0 (0 / eps)
    q = rng.standard_normal((1, 2, 9, D))
    k = -np.abs(rng.standard_normal((1, 2, 9, D))) - 0.1
    v = rng.standard_normal((1, 2, 9, D))
    o = impl.linattn(q, k, v, EPS)
    assert np.all(o == 0.0), "all-negative keys must give exact zeros"
    # all queries negative -> exact zeros
    o = impl.linattn(-np.abs(q) - 0.1, rng.standard_normal(k.shape), v, EPS)
    assert np.all(o == 0.0), "all-negative queries must give exact zeros"
    # D = 1: scalars
    q, k, v = (rng.standard_normal((1, 1, 12, 1)) for _ in range(3))
    rk = np.maximum(k[0, 0, :, 0], 0)
    rq = np.maximum(q[0, 0, :, 0], 0)
    want = rq * np.dot(rk, v[0, 0, :, 0]) / (rq * rk.sum() + EPS)
    _close(impl.linattn(q, k, v, EPS)[0, 0, :, 0], want, 1e-13, "D=1 scalar form")


def pin_constant_v(impl):
    """Constant V = c gives O_i = c s_i / (s_i + eps) (non-RoPE modes)."""
    rng = np.random.default_rng(22)
    q, k = rng.standard_normal((2, 3, 64, 32)), rng.standard_normal((2, 3, 64, 32))
    c = rng.standard_normal(32)
    v = np.broadcast_to(c, q.shape).copy()
    s = np.maximum(q, 0) @ np.maximum(k, 0).sum(axis=-2)[..., None]
    want = c * s / (s + EPS)
    _close(impl.linattn(q, k, v, EPS), want, 1e-13, "constant V (non-causal)")
    o, _, _ = impl.block_causal(q, k, v, 16, EPS)
    assert np.max(np.abs(o - c)) <= 1e-4 * np.max(np.abs(c)), "constant V (block-causal)"


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def pin_invariants(impl):
    rng = np.random.default_rng(31)
    q, k, v1, v2 = (rng.standard_normal((1, 2, 48, 32)) for _ in range(4))
    # linearity in V
    a, b = 0.75, -1.5
    _close(impl.linattn(q, k, a * v1 + b * v2, EPS),
           a * impl.linattn(q, k, v1, EPS) + b * impl.linattn(q, k, v2, EPS), 1e-12, "linearity in V")
    # joint permutation of (K_j, V_j) leaves the non-causal output unchanged
    perm = rng.permutation(48)
    _close(impl.linattn(q, k[:, :, perm], v1[:, :, perm], EPS), impl.linattn(q, k, v1, EPS), 1e-12,
           "key/value permutation")
    # positive scaling of Q or of K cancels exactly when eps = 0
    _close(impl.linattn(3.0 * q, k, v1, 0.0), impl.linattn(q, k, v1, 0.0), 1e-12, "Q scaling")
    _close(impl.linattn(q, 0.25 * k, v1, 0.0), impl.linattn(q, k, v1, 0.0), 1e-12, "K scaling")
    # the output is a convex combination of V rows per feature (weights >= 0)
    o = impl.linattn(q, k, v1, EPS)
    assert np.all(o <= v1.max(axis=-2, keepdims=True) + 1e-12)
    assert np.all(o >= v1.min(axis=-2, keepdims=True) - 1e-12)


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------

def pin_rope_angles(impl):
    T, Hl, Wl = 3, 4, 5
    ang = impl.rope3d_angles(T, Hl, Wl)
    assert ang.shape == (T * Hl * Wl, 16)

    def n(t, h, w):
        return (t * Hl + h) * Wl + w

    # pair 0 of every axis turns at one radian per step of its coordinate
    assert ang[n(2, 0, 0), 0] == 2.0 and ang[n(0, 3, 0), 4] == 3.0 and ang[n(0, 0, 4), 10] == 4.0
    # t axis: 8 dims, pair k frequency 10000**(-2k/8) = 0.1**k
    _close(ang[n(1, 0, 0), 0:4], [1.0, 0.1, 0.01, 0.001], 1e-14, "t-axis frequencies")
    # h and w axes: 12 dims, pair 3 frequency 10000**(-6/12) = 0.01
    _close(ang[n(0, 1, 0), 7], 0.01, 1e-14, "h-axis pair 3")
    _close(ang[n(0, 0, 1), 13], 0.01, 1e-14, "w-axis pair 3")
    # each axis owns its pairs: t -> 0..3, h -> 4..9, w -> 10..15
    base = ang[n(1, 2, 3)]
    assert np.all(ang[n(2, 2, 3), 4:] == base[4:]) and np.any(ang[n(2, 2, 3), :4] != base[:4])
    assert np.all(ang[n(1, 0, 3), [*range(4), *range(10, 16)]] == base[[*range(4), *range(10, 16)]])
    assert np.all(ang[n(1, 2, 0), :10] == base[:10])
    assert np.all(impl.rope3d_angles(1, 1, 1) == 0.0)


def pin_rope_properties(impl):
    rng = np.random.default_rng(41)
    T, Hl, Wl = 3, 4, 5
    N = T * Hl * Wl
    q, k, v = (rng.standard_normal((1, 2, N, 32)) for _ in range(3))
    # identity rotation (all angles 0) reduces to the plain form
    _close(impl.linattn(q, k, v, EPS, angles=np.zeros((N, 16))), impl.linattn(q, k, v, EPS), 1e-13,
           "identity RoPE")
    # rotation preserves the norm of every pair
    ang = impl.rope3d_angles(T, Hl, Wl)
    x = rng.standard_normal((N, 32))
    r = impl.rotate_pairs(x, ang)
    _close(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), 1e-14, "pair norms")
    # shifting every token's position by the same amount along one axis leaves
    # the output unchanged (the numerator only sees relative rotations)
    big = impl.rope3d_angles(T + 2, Hl + 3, Wl + 1)

    def sub(dt, dh, dw):
        idx = [((t + dt) * (Hl + 3) + (h + dh)) * (Wl + 1) + (w + dw)
               for t in range(T) for h in range(Hl) for w in range(Wl)]
        return big[idx]

    ref = impl.linattn(q, k, v, EPS, angles=sub(0, 0, 0))
    for shift in [(2, 0, 0), (0, 3, 0), (0, 0, 1), (1, 2, 1)]:
        _close(impl.linattn(q, k, v, EPS, angles=sub(*shift)), ref, 1e-11, f"position shift {shift}")
    # the denominator never sees the rotation: O_i * (relu(Q_i).z + eps) is the
    # rotated numerator computed pair by pair from the quadratic definition
    o = impl.linattn(q, k, v, EPS, angles=ang)
    pq, pk = np.maximum(q, 0), np.maximum(k, 0)
    den = pq @ pk.sum(axis=-2)[..., None] + EPS
    R = np.zeros((N, 32, 32))
    for p in range(16):
        c, s = np.cos(ang[:, p]), np.sin(ang[:, p])
        R[:, 2 * p, 2 * p], R[:, 2 * p, 2 * p + 1] = c, -s
        R[:, 2 * p + 1, 2 * p], R[:, 2 * p + 1, 2 * p + 1] = s, c
    rq = np.einsum("nij,bhnj->bhni", R, pq)
    rk = np.einsum("nij,bhnj->bhni", R, pk)
    _close(o * den, (rq @ np.swapaxes(rk, -1, -2)) @ v, 1e-11, "un-rotated denominator")


# --------------------------------------------------------------------------
# Block-causal properties
# --------------------------------------------------------------------------

def pin_block_properties(impl):
    rng = np.random.default_rng(51)
    N, L = 50, 12
    q, k, v = (rng.standard_normal((2, 2, N, 32)) for _ in range(3))
    o, S, z = impl.block_causal(q, k, v, L, EPS)
    # one chunk covering everything is the non-causal form
    o1, _, _ = impl.block_causal(q, k, v, N, EPS)
    _close(o1, impl.linattn(q, k, v, EPS), 1e-12, "single chunk == non-causal")
    # the last chunk's rows see everything: equal to the non-causal rows
    last = slice((N - 1) // L * L, N)
    _close(o[:, :, last], impl.linattn(q, k, v, EPS)[:, :, last], 1e-12, "last chunk == non-causal rows")
    # the first chunk sees only itself
    _close(o[:, :, :L], impl.linattn(q[:, :, :L], k[:, :, :L], v[:, :, :L], EPS), 1e-12,
           "first chunk == its own non-causal attention")
    # the final carried state is the full-sequence state
    S_full, z_full = impl.kv_state(k, v)
    _close(S, S_full, 1e-12, "final S")
    _close(z, z_full, 1e-12, "final z")
    # causality: changing chunk 2 onwards leaves chunks 0..1 bit-identical
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, :, 2 * L:] = rng.standard_normal(x[:, :, 2 * L:].shape)
    o2, _, _ = impl.block_causal(q2, k2, v2, L, EPS)
    assert np.array_equal(o2[:, :, :2 * L], o[:, :, :2 * L]), "earlier chunks saw a later chunk"
    assert not np.array_equal(o2[:, :, 2 * L:3 * L], o[:, :, 2 * L:3 * L])
    # save / restore of the carried state mid-sequence is bit-identical
    S_c = np.zeros((2, 2, 32, 32))
    z_c = np.zeros((2, 2, 32))
    outs = []
    for c, start in enumerate(range(0, N, L)):
        sl = slice(start, min(N, start + L))
        if c == 2:
            S_c, z_c = np.array(S_c.tolist()), np.array(z_c.tolist())   # round trip through host lists
        oc, S_c, z_c = impl.block_forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], S_c, z_c, EPS)
        outs.append(oc)
    assert np.array_equal(np.concatenate(outs, axis=2), o), "save/restore changed the result"
    # state_update applied in two pieces equals one call
    Sa, za = impl.state_update(k[:, :, :20], v[:, :, :20], np.zeros_like(S), np.zeros_like(z))
    Sa, za = impl.state_update(k[:, :, 20:], v[:, :, 20:], Sa, za, None, 20)
    _close(Sa, S_full, 1e-12, "two-piece state_update S")
    _close(za, z_full, 1e-12, "two-piece state_update z")


def pin_block_rope_positions(impl):
    """Block mode with RoPE indexes the angle table by global token position."""
    rng = np.random.default_rng(52)
    T, Hl, Wl = 2, 3, 4
    N, L = T * Hl * Wl, 5
    ang = impl.rope3d_angles(T, Hl, Wl)
    q, k, v = (rng.standard_normal((1, 1, N, 32)) for _ in range(3))
    o, _, _ = impl.block_causal(q, k, v, L, EPS, angles=ang)
    _close(o, impl.brute_force(q, k, v, EPS, angles=ang, chunk=L), 1e-11, "block RoPE vs masked quadratic")


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def pin_backward_exact(impl):
    """The state-form gradients against the exact gradients of the quadratic
    definition (differentiated directly, in rational arithmetic)."""
    rng = np.random.default_rng(61)
    for N, D, L, rope in [(3, 2, None, False), (5, 4, 2, False), (7, 4, 1, False), (4, 4, None, True),
                          (6, 4, 3, True), (5, 6, 5, False)]:
        q, k, v, do = (_dyadic(rng, (N, D)) for _ in range(4))
        ang = rng.uniform(-3.0, 3.0, size=(N, D // 2)) if rope else None
        cs = (np.cos(ang), np.sin(ang)) if rope else (None, None)
        want = exact_gradients(q, k, v, do, EPS, *cs, chunk=L)
        got = impl.backward(q[None, None], k[None, None], v[None, None], do[None, None], EPS, angles=ang, chunk=L)
        for g, w, name in zip(got[:3], want, ("dq", "dk", "dv")):
            _close(g[0, 0], w, 1e-8, f"{name} vs exact quadratic-form gradient N={N} D={D} chunk={L} rope={rope}")


def _away_from_zero(rng, shape):
    """Normal draws pushed at least 0.2 away from 0, so that a finite-difference
    step never crosses the ReLU kink."""
    x = rng.standard_normal(shape)
    return x + 0.2 * np.sign(x)


def pin_backward_finite_differences(impl):
    """Central differences of the forward (chunk by chunk through block_forward,
    from a carried state, plus <dS_out, S_out> + dz_out . z_out) against every
    gradient the backward returns, including those of the carried state."""
    rng = np.random.default_rng(62)
    T, Hl, Wl = 2, 2, 3
    N, D, L = T * Hl * Wl, 8, 5
    ang = impl.rope3d_angles(T, Hl, Wl, D=D, split=(2, 2, 4))
    x = {n: _away_from_zero(rng, (N, D)) for n in ("q", "k", "v", "do")}
    S_in, z_in = rng.standard_normal((D, D)), np.abs(rng.standard_normal(D)) + 0.5
    dS_out, dz_out = rng.standard_normal((D, D)), rng.standard_normal(D)

    def loss(q, k, v, S, z):
        total = 0.0
        for start in range(0, N, L):
            sl = slice(start, min(N, start + L))
            o, S, z = impl.block_forward(q[sl][None, None], k[sl][None, None], v[sl][None, None], S[None, None],
                                         z[None, None], EPS, ang, start)
            o, S, z = o[0, 0], S[0, 0], z[0, 0]
            total += float((x["do"][sl] * o).sum())
        return total + float((dS_out * S).sum()) + float((dz_out * z).sum())

    got = impl.backward(x["q"][None, None], x["k"][None, None], x["v"][None, None], x["do"][None, None], EPS,
                        angles=ang, chunk=L, S_in=S_in[None, None], z_in=z_in[None, None],
                        dS_out=dS_out[None, None], dz_out=dz_out[None, None])
    grads = {"q": got[0][0, 0], "k": got[1][0, 0], "v": got[2][0, 0], "S": got[3][0, 0], "z": got[4][0, 0]}
    args = {"q": x["q"], "k": x["k"], "v": x["v"], "S": S_in, "z": z_in}
    h = 1e-5
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = {n: a.copy() for n, a in args.items()}
            minus = {n: a.copy() for n, a in args.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            fd[idx] = (loss(**plus) - loss(**minus)) / (2 * h)
        _close(grads[name], fd, 1e-6, f"d{name} vs central differences of the forward")


ALL_PINS = [
    pin_exact_noncausal, pin_exact_state, pin_exact_rope, pin_exact_block, pin_exact_block_rope,
    pin_token_causal, pin_closed_forms, pin_constant_v, pin_invariants, pin_rope_angles,
    pin_rope_properties, pin_block_properties, pin_block_rope_positions,
    pin_backward_exact, pin_backward_finite_differences,
]


# --------------------------------------------------------------------------
# Temporal convolution (block-inference conv cache)
# --------------------------------------------------------------------------

def pin_temporal_conv(impl):
    """Against a loop over frames written from the formula, exact in
    rationals for dyadic inputs; chunking with the cache equals one pass over
    the whole sequence except at the chunk ends (no look-ahead across chunks);
    identity and shift filters."""
    from fractions import Fraction
    rng = np.random.default_rng(71)
    B, F, S, C = 2, 4, 3, 5
    x = _dyadic(rng, (B, F, S, C))
    w = _dyadic(rng, (C, 3))
    b = _dyadic(rng, (C,))
    prev = _dyadic(rng, (B, S, C))
    y, cache = impl.temporal_conv3(x, w, b, prev)
    for bb in range(B):
        for f in range(F):
            for s in range(S):
                for c in range(C):
                    left = prev[bb, s, c] if f == 0 else x[bb, f - 1, s, c]
                    right = 0.0 if f == F - 1 else x[bb, f + 1, s, c]
                    want = (Fraction(x[bb, f, s, c]) + Fraction(w[c, 0]) * Fraction(left)
                            + Fraction(w[c, 1]) * Fraction(x[bb, f, s, c]) + Fraction(w[c, 2]) * Fraction(right)
                            + Fraction(b[c]))
                    assert y[bb, f, s, c] == float(want), (bb, f, s, c)
    assert np.array_equal(cache, x[:, F - 1])
    # the first chunk starts from zeros
    y0, _ = impl.temporal_conv3(x, w, b, None)
    y1, _ = impl.temporal_conv3(x, w, b, np.zeros((B, S, C)))
    assert np.array_equal(y0, y1)
    # chunks of 2 frames with the cache: frame 1 of each chunk misses only its right neighbour
    ya, ca = impl.temporal_conv3(x[:, :2], w, b, prev)
    yb, cb = impl.temporal_conv3(x[:, 2:], w, b, ca)
    _close(ya[:, 0], y[:, 0], 0.0, "first frame")
    _close(yb, y[:, 2:], 0.0, "second chunk through the cache")
    _close(ya[:, 1] + w[:, 2] * x[:, 2], y[:, 1], 1e-15, "chunk end: no later frame")
    assert np.array_equal(cb, cache)
    # w = (0, 0, 0) and no bias: the shortcut alone; w = (1, -1, 0): y = x_prev
    z, _ = impl.temporal_conv3(x, np.zeros((C, 3)), None, prev)
    assert np.array_equal(z, x)
    sh = np.tile(np.array([1.0, -1.0, 0.0]), (C, 1))
    z, _ = impl.temporal_conv3(x, sh, None, prev)
    assert np.array_equal(z[:, 0], prev) and np.array_equal(z[:, 1:], x[:, :-1])


ALL_PINS.append(pin_temporal_conv)


# --------------------------------------------------------------------------
# Key/value projection feeding the state
# --------------------------------------------------------------------------

def _bf16_by_bits(x32):
    """Round float32 values to bfloat16 through their bit patterns: add
    0x7fff plus the lowest kept bit, then clear the 16 low bits (round to
    nearest, ties to even)."""
    bits = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    kept = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return kept.astype(np.uint32).view(np.float32).astype(np.float64)


def pin_projected_state(impl):
    """bf16 rounding against the bit-pattern method and hand-made ties; the
    projected state against a brute-force loop in rationals (rounding written
    as a search over the two neighbouring bf16 values), plain and with keys
    rotated by explicit 2 x 2 rotations at offset positions; identity weights
    reduce it to kv_state of the input; doubling the input quadruples S."""
    from fractions import Fraction
    rng = np.random.default_rng(81)
    x32 = (rng.standard_normal(4000) * np.float32(3.0)).astype(np.float32)
    assert np.array_equal(impl.round_bf16(x32.astype(np.float64)), _bf16_by_bits(x32))
    # ties go to the even neighbour; just above a tie rounds up
    assert impl.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert impl.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert impl.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert impl.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -20)) == -(1.0 + 2.0 ** -7)

    def rb_fraction(f):
        # the nearest value with 8 significant bits, ties to an even last bit
        if f == 0:
            return Fraction(0)
        sign = 1 if f > 0 else -1
        a = abs(f)
        e = 0
        while a >= 2:
            a /= 2
            e += 1
        while a < 1:
            a *= 2
            e -= 1
        lo = Fraction(int(a * 128), 128)
        hi = lo + Fraction(1, 128)
        d_lo, d_hi = a - lo, hi - a
        pick = lo if d_lo < d_hi else hi if d_hi < d_lo else (lo if (lo * 128) % 2 == 0 else hi)
        return sign * pick * Fraction(2) ** e

    # bf16 inputs with full 8-bit mantissas, so the projections need rounding
    B, H, N, C, D = 1, 2, 5, 6, 3
    x = _bf16_by_bits(rng.standard_normal((B, N, C)).astype(np.float32))
    wk = _bf16_by_bits(rng.standard_normal((H, C, D)).astype(np.float32))
    wv = _bf16_by_bits(rng.standard_normal((H, C, D)).astype(np.float32))
    raw = np.matmul(x[:, None], wk[None])
    assert np.any(raw != _bf16_by_bits(raw.astype(np.float32))), "the case must exercise the rounding"
    S, z = impl.projected_kv_state(x, wk, wv)
    assert S.shape == (B, H, D, D) and z.shape == (B, H, D)
    for h in range(H):
        K = [[rb_fraction(sum(Fraction(x[0, n, c]) * Fraction(wk[h, c, d]) for c in range(C))) for d in range(D)]
             for n in range(N)]
        V = [[rb_fraction(sum(Fraction(x[0, n, c]) * Fraction(wv[h, c, e]) for c in range(C))) for e in range(D)]
             for n in range(N)]
        for d in range(D):
            assert z[0, h, d] == float(sum(max(K[n][d], 0) for n in range(N))), ("z", h, d)
            for e in range(D):
                want = sum(max(K[n][d], 0) * V[n][e] for n in range(N))
                assert S[0, h, d, e] == float(want), ("S", h, d, e)
    # identity weights: the projection is the input itself (bf16-exact)
    xi = np.asarray(impl.round_bf16(rng.standard_normal((2, 7, 4))), dtype=np.float64)
    eye = np.broadcast_to(np.eye(4), (3, 4, 4))
    S_i, z_i = impl.projected_kv_state(xi, eye, eye)
    S_k, z_k = impl.kv_state(np.broadcast_to(xi[:, None], (2, 3, 7, 4)), np.broadcast_to(xi[:, None], (2, 3, 7, 4)))
    assert np.array_equal(S_i, S_k) and np.array_equal(z_i, z_k)
    # a power-of-two scale commutes with the rounding: S scales by 4, z by 2
    S2, z2 = impl.projected_kv_state(2.0 * x, wk, wv)
    assert np.array_equal(S2, 4.0 * S) and np.array_equal(z2, 2.0 * z)

    # rotated keys: the brute force again, each key's pairs (2p, 2p + 1) turned
    # by an explicit 2 x 2 rotation in rationals from the float64 cos and sin
    # of its position's angles (positions pos_offset + n); z stays unrotated
    D2 = 4
    wk2 = _bf16_by_bits(rng.standard_normal((H, C, D2)).astype(np.float32))
    wv2 = _bf16_by_bits(rng.standard_normal((H, C, D2)).astype(np.float32))
    angles = rng.uniform(-3.0, 3.0, (N + 3, D2 // 2))
    S_r, z_r = impl.projected_kv_state(x, wk2, wv2, angles=angles, pos_offset=2)
    _, z_plain = impl.projected_kv_state(x, wk2, wv2)
    assert np.array_equal(z_r, z_plain)
    for h in range(H):
        K = [[rb_fraction(sum(Fraction(x[0, n, c]) * Fraction(wk2[h, c, d]) for c in range(C))) for d in range(D2)]
             for n in range(N)]
        V = [[rb_fraction(sum(Fraction(x[0, n, c]) * Fraction(wv2[h, c, e]) for c in range(C))) for e in range(D2)]
             for n in range(N)]
        for d in range(D2):
            for e in range(D2):
                want = Fraction(0)
                for n in range(N):
                    p = d // 2
                    cs, sn = Fraction(np.cos(angles[n + 2, p])), Fraction(np.sin(angles[n + 2, p]))
                    k0, k1 = max(K[n][2 * p], 0), max(K[n][2 * p + 1], 0)
                    rot = k0 * cs - k1 * sn if d % 2 == 0 else k0 * sn + k1 * cs
                    want += rot * V[n][e]
                assert abs(S_r[0, h, d, e] - float(want)) <= 1e-12 * (1 + abs(float(want))), ("S rotated", h, d, e)


ALL_PINS.append(pin_projected_state)


def pin_projected_apply(impl):
    """The projected queries' outputs against a brute force in rationals: the
    query projection rounded by search, its ReLU, the numerator with explicit
    2 x 2 rotations at offset positions and the unrotated denominator, each
    output one rational division; identity weights reduce it to apply_state of
    the input; a positive power-of-two scale of the input leaves O unchanged at
    eps = 0."""
    from fractions import Fraction
    rng = np.random.default_rng(91)

    def rb_fraction(f):
        if f == 0:
            return Fraction(0)
        sign = 1 if f > 0 else -1
        a, e = abs(f), 0
        while a >= 2:
            a /= 2
            e += 1
        while a < 1:
            a *= 2
            e -= 1
        lo = Fraction(int(a * 128), 128)
        hi = lo + Fraction(1, 128)
        d_lo, d_hi = a - lo, hi - a
        pick = lo if d_lo < d_hi else hi if d_hi < d_lo else (lo if (lo * 128) % 2 == 0 else hi)
        return sign * pick * Fraction(2) ** e

    B, H, N, C, D = 1, 2, 4, 5, 4
    x = _bf16_by_bits(rng.standard_normal((B, N, C)).astype(np.float32))
    wq = _bf16_by_bits(rng.standard_normal((H, C, D)).astype(np.float32))
    S = rng.standard_normal((B, H, D, D))
    z = rng.uniform(0.5, 2.0, (B, H, D))
    angles = rng.uniform(-3.0, 3.0, (N + 2, D // 2))
    eps = 1e-3
    raw = np.matmul(x[:, None], wq[None])
    assert np.any(raw != _bf16_by_bits(raw.astype(np.float32))), "the case must exercise the rounding"
    for ang, off in ((None, 0), (angles, 2)):
        O = impl.projected_apply(x, wq, S, z, eps, angles=ang, pos_offset=off)
        assert O.shape == (B, H, N, D)
        for h in range(H):
            for n in range(N):
                Q = [max(rb_fraction(sum(Fraction(x[0, n, c]) * Fraction(wq[h, c, d]) for c in range(C))), 0)
                     for d in range(D)]
                den = sum(Q[d] * Fraction(z[0, h, d]) for d in range(D)) + Fraction(eps)
                if ang is None:
                    R = Q
                else:
                    R = []
                    for d in range(D):
                        p = d // 2
                        cs, sn = Fraction(np.cos(ang[n + off, p])), Fraction(np.sin(ang[n + off, p]))
                        q0, q1 = Q[2 * p], Q[2 * p + 1]
                        R.append(q0 * cs - q1 * sn if d % 2 == 0 else q0 * sn + q1 * cs)
                for e in range(D):
                    want = float(sum(R[d] * Fraction(S[0, h, d, e]) for d in range(D)) / den)
                    assert abs(O[0, h, n, e] - want) <= 1e-12 * (1 + abs(want)), ("O", ang is None, h, n, e)
    # identity weights: the projection is the input itself (bf16-exact)
    xi = np.asarray(impl.round_bf16(rng.standard_normal((1, 6, 4))), dtype=np.float64)
    eye = np.broadcast_to(np.eye(4), (2, 4, 4))
    Si = rng.standard_normal((1, 2, 4, 4))
    zi = rng.uniform(0.5, 2.0, (1, 2, 4))
    got = impl.projected_apply(xi, eye, Si, zi, 1e-6)
    want = impl.apply_state(np.broadcast_to(xi[:, None], (1, 2, 6, 4)), Si, zi, 1e-6)
    assert np.array_equal(got, want)
    # numerator and denominator are both linear in phi(Q): a power-of-two scale
    # cancels exactly at eps = 0 (rows with phi(Q) = 0 are 0/0 in both)
    with np.errstate(invalid="ignore", divide="ignore"):
        O1 = impl.projected_apply(x, wq, S, z, 0.0)
        O4 = impl.projected_apply(4.0 * x, wq, S, z, 0.0)
    assert np.count_nonzero(np.isfinite(O1)) > O1.size // 2
    assert np.array_equal(O1, O4, equal_nan=True)


ALL_PINS.append(pin_projected_apply)
