"""Exact rational (fractions.Fraction) brute force of the attention definitions.

Independent of NumPy and of the oracle: it evaluates the softmax-free
quadratic forms token pair by token pair, for tiny inputs only.  Floats are
converted to Fractions exactly, so the only rounding left is the final
conversion back to float.

Definitions (SANA-Video paper notes, sections 2.1-2.3; SANA-Video news
article, "Design details"):
  non-causal  O_i = sum_j A_ij V_j / (sum_j A_ij + eps),  A_ij = relu(Q_i).relu(K_j)
  RoPE        numerator weights use (R_i relu(Q_i)).(R_j relu(K_j)),
              the denominator keeps A_ij
  block       only pairs with chunk(j) <= chunk(i) take part
"""

from fractions import Fraction


def _relu(x):
    return x if x > 0 else Fraction(0)


def _frac_rows(rows):
    return [[Fraction(float(x)) for x in row] for row in rows]


def _rotation_matrix(cos_row, sin_row):
    """Explicit D x D block-diagonal rotation: block p = [[c, -s], [s, c]] on (2p, 2p+1)."""
    D = 2 * len(cos_row)
    R = [[Fraction(0)] * D for _ in range(D)]
    for p, (c, s) in enumerate(zip(cos_row, sin_row)):
        R[2 * p][2 * p] = c
        R[2 * p][2 * p + 1] = -s
        R[2 * p + 1][2 * p] = s
        R[2 * p + 1][2 * p + 1] = c
    return R


def _matvec(R, x):
    return [sum((R[r][c] * x[c] for c in range(len(x))), Fraction(0)) for r in range(len(R))]


def exact_attention(q, k, v, eps, cos=None, sin=None, chunk=None):
    """q, k, v: [N][D] float-likes; cos, sin: [N][D/2] float-likes or None.

    Returns [N][D] floats.
    """
    Q, K, V = _frac_rows(q), _frac_rows(k), _frac_rows(v)
    eps = Fraction(float(eps))
    N, D = len(Q), len(Q[0])
    pq = [[_relu(x) for x in row] for row in Q]
    pk = [[_relu(x) for x in row] for row in K]
    if cos is not None:
        C, S = _frac_rows(cos), _frac_rows(sin)
        rq = [_matvec(_rotation_matrix(C[i], S[i]), pq[i]) for i in range(N)]
        rk = [_matvec(_rotation_matrix(C[j], S[j]), pk[j]) for j in range(N)]
    out = []
    for i in range(N):
        num = [Fraction(0)] * D
        den = Fraction(0)
        for j in range(N):
            if chunk is not None and j // chunk > i // chunk:
                continue
            a = sum((pq[i][d] * pk[j][d] for d in range(D)), Fraction(0))
            if cos is None:
                a_num = a
            else:
                a_num = sum((rq[i][d] * rk[j][d] for d in range(D)), Fraction(0))
            den += a
            for e in range(D):
                num[e] += a_num * V[j][e]
        out.append([float(num[e] / (den + eps)) if den + eps != 0 else float("nan")
                    for e in range(D)])
    return out


def exact_state(k, v):
    """Exact (S, z): S[d][e] = sum_j relu(K_jd) V_je, z[d] = sum_j relu(K_jd)."""
    K, V = _frac_rows(k), _frac_rows(v)
    D = len(K[0])
    S = [[sum((_relu(K[j][d]) * V[j][e] for j in range(len(K))), Fraction(0)) for e in range(D)]
         for d in range(D)]
    z = [sum((_relu(K[j][d]) for j in range(len(K))), Fraction(0)) for d in range(D)]
    return [[float(x) for x in row] for row in S], [float(x) for x in z]


def token_causal_recurrence(q, k, v, eps):
    """Token-by-token causal recurrence (inclusive): the running sums after token
    i are applied to token i's query.  Exact arithmetic, loops only."""
    Q, K, V = _frac_rows(q), _frac_rows(k), _frac_rows(v)
    eps = Fraction(float(eps))
    N, D = len(Q), len(Q[0])
    S = [[Fraction(0)] * D for _ in range(D)]
    z = [Fraction(0)] * D
    out = []
    for i in range(N):
        for d in range(D):
            kd = _relu(K[i][d])
            z[d] += kd
            for e in range(D):
                S[d][e] += kd * V[i][e]
        pq = [_relu(x) for x in Q[i]]
        den = sum((pq[d] * z[d] for d in range(D)), Fraction(0)) + eps
        out.append([float(sum((pq[d] * S[d][e] for d in range(D)), Fraction(0)) / den)
                    for e in range(D)])
    return out


def _transpose(R):
    return [list(row) for row in zip(*R)]


def exact_gradients(q, k, v, dout, eps, cos=None, sin=None, chunk=None):
    """Gradients of L = sum_i dout_i . O_i, differentiating the quadratic
    definition above directly (not its linear/state form), exactly.

      O_i = Num_i / d_i,  Num_i = sum_j M_ij A'_ij V_j,  d_i = sum_j M_ij A_ij + eps
      dL/dV_j   = sum_i M_ij A'_ij dout_i / d_i
      dL/dA'_ij = M_ij (dout_i . V_j) / d_i
      dL/dA_ij  = -M_ij (dout_i . Num_i) / d_i^2
      A'_ij = (R_i p_i).(R_j r_j): gradient R_i^T R_j r_j in p_i, R_j^T R_i p_i in r_j
      A_ij  = p_i . r_j,  p = relu(Q), r = relu(K);  dQ = [Q > 0] dL/dp, dK = [K > 0] dL/dr.

    Returns (dq, dk, dv) as [N][D] floats.
    """
    Q, K, V, G = _frac_rows(q), _frac_rows(k), _frac_rows(v), _frac_rows(dout)
    eps = Fraction(float(eps))
    N, D = len(Q), len(Q[0])
    pq = [[_relu(x) for x in row] for row in Q]
    pk = [[_relu(x) for x in row] for row in K]
    if cos is not None:
        C, S = _frac_rows(cos), _frac_rows(sin)
        R = [_rotation_matrix(C[i], S[i]) for i in range(N)]
        rq = [_matvec(R[i], pq[i]) for i in range(N)]
        rk = [_matvec(R[j], pk[j]) for j in range(N)]
    else:
        rq, rk = pq, pk

    def seen(i, j):
        return chunk is None or j // chunk <= i // chunk

    num, den = [], []
    for i in range(N):
        n_i = [Fraction(0)] * D
        d_i = eps
        for j in range(N):
            if not seen(i, j):
                continue
            a = sum((pq[i][d] * pk[j][d] for d in range(D)), Fraction(0))
            a_num = sum((rq[i][d] * rk[j][d] for d in range(D)), Fraction(0))
            d_i += a
            for e in range(D):
                n_i[e] += a_num * V[j][e]
        num.append(n_i)
        den.append(d_i)

    dp = [[Fraction(0)] * D for _ in range(N)]
    dr = [[Fraction(0)] * D for _ in range(N)]
    dV = [[Fraction(0)] * D for _ in range(N)]
    for i in range(N):
        g_dot_num = sum((G[i][e] * num[i][e] for e in range(D)), Fraction(0))
        for j in range(N):
            if not seen(i, j):
                continue
            a_num = sum((rq[i][d] * rk[j][d] for d in range(D)), Fraction(0))
            for e in range(D):
                dV[j][e] += a_num * G[i][e] / den[i]
            g_a_num = sum((G[i][e] * V[j][e] for e in range(D)), Fraction(0)) / den[i]
            g_a = -g_dot_num / (den[i] * den[i])
            if cos is not None:
                to_p = _matvec(_transpose(R[i]), rk[j])   # R_i^T R_j r_j
                to_r = _matvec(_transpose(R[j]), rq[i])   # R_j^T R_i p_i
            else:
                to_p, to_r = pk[j], pq[i]
            for d in range(D):
                dp[i][d] += g_a_num * to_p[d] + g_a * pk[j][d]
                dr[j][d] += g_a_num * to_r[d] + g_a * pq[i][d]
    dq = [[float(dp[i][d]) if Q[i][d] > 0 else 0.0 for d in range(D)] for i in range(N)]
    dk = [[float(dr[j][d]) if K[j][d] > 0 else 0.0 for d in range(D)] for j in range(N)]
    dv = [[float(x) for x in row] for row in dV]
    return dq, dk, dv
