"""Element-wise error bound for the fused key/value projection and state
update, against the float64 oracle's projected_kv_state.

The bound, derived from the arithmetic.  The kernel sums a projection as
C / 32 MFMA steps of 32 products each, in fp32: whatever the order inside a
step, a product passes through at most 31 + C / 32 roundings, so the fp32
value lies within delta = 2 (C / 32 + 32) 2^-24 sum_c |x_c w_c| of the exact
one (the factor 2 also covers truncating adders).  Rounding to bf16 is
monotone, so the kernel's K lies between round(K - delta) and
round(K + delta), b_K apart: 0 unless K sits next to a rounding boundary, then
one bf16 step.  The state's fp32 sums pass each product through at most
31 + N / 32 + (partials) + 2 roundings, bounded by N / 32 + 200.  So, with
A = |phi(K)|^T |V| over the tokens (the b's added in),
  |dS| <= b_K^T (|V| + b_V) + |phi(K)|^T b_V + 2 (N / 32 + 200) 2^-24 A,
  |dz| <= sum b_K + 2 (N / 32 + 200) 2^-24 sum (|phi(K)| + b_K),
plus, when the call starts from a carried state S0 (z0), the same factor times
|S0| (|z0|): it is the first term of those sums.
With RoPE, S contracts the rotated keys y = R phi(K): y_d = x_d c -+ x_d' s
(d' = d ^ 1), taken in fp32 from float32 cos/sin and split into three bf16
parts.  Against the oracle's float64 rotation, |dy_d| <= b_d + b_d' +
6 2^-24 (|x_d| + |x_d'| + b_d + b_d') (|c|, |s| <= 1: two products and a sum,
the float32 rounding of cos and sin, the split's remainder), and the bound
above holds with y and dy in place of phi(K) and b_K in S, and 3 N / 32 in
place of N / 32 (three parts added per 32 tokens); z stays unrotated.
A relative-error bar would not do: one K rounding the other way moves an
element of S that happens to be near zero by far more than a fixed fraction of
it.  The aggregate rel-L2 must also stay below 1e-3.  A library GEMM of
unknown summation order (the unfused path) gets delta = 2 C 2^-24 instead."""

import numpy as np

import oracle
from metrics import BF16_MAX_REL, BF16_REL_L2, FLOOR, rel_l2

REL_L2 = 1e-3
U = 2.0 ** -24


def oracle_weights(w, H, D=32):
    """[H*D, C] rows (a linear layer's weight) -> the oracle's [H, C, D]."""
    C = w.shape[1]
    return np.ascontiguousarray(w.reshape(H, D, C).transpose(0, 2, 1))


def _spread(x, w, any_order=False):
    """bf16(x w) for x [B, N, C] and w [H', C, 32], and the width b of its
    rounding interval: the fp32 sum lies within delta of the exact value, so
    the kernel's bf16 value lies between round(exact - delta) and
    round(exact + delta)."""
    C = x.shape[-1]
    exact = np.matmul(x[:, None], w[None])                     # [B, H', N, 32]
    steps = C if any_order else C / 32 + 32
    delta = 2.0 * steps * U * np.matmul(np.abs(x)[:, None], np.abs(w)[None])
    lo, hi = oracle.round_bf16(exact - delta), oracle.round_bf16(exact + delta)
    return oracle.round_bf16(exact), hi - lo, lo, hi


def check_projected_state(kv, z, x, heads=None, kv0=None, z0=None, any_order=False, angles=None, pos_offset=0):
    """kv, z (float64, [B, H', 32, 32] and [B, H', 32] for the chosen heads of
    the ProjectionInputs x) against the oracle within the bound above, with
    kv0, z0 the states the call started from (None: zero).  any_order: the
    projection's sums were taken in an unknown order.  angles, pos_offset: the
    keys' RoPE, as for the oracle.  Returns (ok, report)."""
    p = x.workload
    wk, wv = oracle_weights(x.f64["w_k"], p.H), oracle_weights(x.f64["w_v"], p.H)
    if heads is not None:
        wk, wv = wk[heads], wv[heads]
    S, zr = oracle.projected_kv_state(x.f64["x"], wk, wv, angles, pos_offset)
    if kv0 is not None:
        S, zr = S + kv0, zr + z0
    N = p.N

    def spread(w):
        q, b, _lo, _hi = _spread(x.f64["x"], w, any_order)
        return q, b

    K, bK = spread(wk)
    V, bV = spread(wv)
    phik = np.maximum(K, 0.0)
    absV = np.abs(V) + bV
    if angles is None:
        Y, bY = phik, bK
    else:
        Y = np.abs(oracle.rotate_pairs(phik, angles[pos_offset:pos_offset + N]))
        sw = np.arange(phik.shape[-1]) ^ 1                      # pair partner of each feature
        bY = bK + bK[..., sw] + 6.0 * U * (phik + phik[..., sw] + bK + bK[..., sw])
    yt = np.swapaxes(np.abs(Y), -1, -2)
    byt = np.swapaxes(bY, -1, -2)
    # with RoPE each 32-token group adds three parts to the accumulator
    gam = 2.0 * ((1 if angles is None else 3) * N / 32 + 200) * U
    tol_S = np.matmul(byt, absV) + np.matmul(yt, bV) + gam * np.matmul(yt + byt, absV)
    tol_z = bK.sum(axis=-2) + gam * (phik + bK).sum(axis=-2)
    if kv0 is not None:
        # the carried state enters the same fp32 sums: each rounding is relative
        # to the running total, which includes it
        tol_S = tol_S + gam * np.abs(kv0)
        tol_z = tol_z + gam * np.abs(z0)
    n_amb = int(np.count_nonzero(bK)) + int(np.count_nonzero(bV))
    lines = []
    for got, want, tol, name in ((kv, S, tol_S, "S"), (z, zr, tol_z, "z")):
        got = np.asarray(got, dtype=np.float64)
        err = np.abs(got - want)
        l2 = rel_l2(got, want)
        worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
        lines.append(f"{name}: rel-L2 {l2:.3e}, max |err| / bound {worst:.3e} "
                     f"({n_amb} of {K.size + V.size} projected values next to a rounding boundary)")
        if not np.all(np.isfinite(got)):
            return False, lines[-1] + ": non-finite output"
        if l2 > REL_L2:
            return False, lines[-1] + ": rel-L2 above 1e-3"
        if not np.all(err <= tol):
            return False, lines[-1] + ": error above the derived bound"
    return True, "\n".join(lines)


def check_projected_apply(o, x, S, z, eps, heads=None, angles=None, pos_offset=0, any_order=False):
    """o (float64 [B, H', N, 32], the chosen heads of the ProjectionInputs x,
    with w_q) against the oracle's projected_apply with states S, z.

    The output is o_e = sum_d y_d S_de / (sum_d p_d z_d + eps), p = phi(Q), y
    = p or its RoPE rotation R p.  Where a feature of Q is next to a bf16
    rounding boundary (the interval of _spread), the kernel may hold the other
    neighbour: p_f moves by at most b_f = relu(hi_f) - relu(lo_f) (one bf16
    step, or less across zero), and o_e by b_f |d o_e / d p_f| <= b_f (|S_fe|
    (+ |S_f'e|, f' = f ^ 1, under the rotation) + |o_e| z_f) / den, to first
    order; the factor 1.5 covers the second-order term (b_f / p_f <= 2^-7).
    Elsewhere the bf16 bar holds: |err_e| <= 2e-2 max(|o_e|, 1e-3 rms(o)),
    plus the ambiguity term; the rel-L2 over the whole output stays <= 4e-3.
    any_order: Q's sums were taken in an unknown order.  Returns (ok, report)."""
    p = x.workload
    wq = oracle_weights(x.f64["w_q"], p.H)
    S = np.asarray(S, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    if heads is not None:
        wq, S, z = wq[heads], S[:, heads], z[:, heads]
    want = oracle.projected_apply(x.f64["x"], wq, S, z, eps, angles, pos_offset)
    Q, _b, lo, hi = _spread(x.f64["x"], wq, any_order)
    bp = np.maximum(hi, 0.0) - np.maximum(lo, 0.0)               # [B, H', N, 32]
    den = np.matmul(np.maximum(Q, 0.0), z[..., :, None]) + eps  # [B, H', N, 1]
    Sa = np.abs(S)
    if angles is not None:
        Sa = Sa + Sa[..., np.arange(Sa.shape[-2]) ^ 1, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        amb = 1.5 * (np.matmul(bp, Sa) + np.abs(want) * np.matmul(bp, z[..., :, None])) / den
    amb = np.where(np.isfinite(amb), amb, np.inf)
    o = np.asarray(o, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want * want))) if want.size else 0.0
    tol = BF16_MAX_REL * np.maximum(np.abs(want), FLOOR * rms) + amb
    err = np.abs(o - want)
    l2 = rel_l2(o, want)
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    report = (f"rel-L2 {l2:.3e}, max |err| / bound {worst:.3e} ({int(np.count_nonzero(bp))} of {bp.size} "
              f"query features next to a rounding boundary)")
    if not np.all(np.isfinite(o)):
        return False, report + ": non-finite output"
    if l2 > BF16_REL_L2:
        return False, report + ": rel-L2 above 4e-3"
    if not np.all(err <= tol):
        return False, report + ": error above the bound"
    return True, report
