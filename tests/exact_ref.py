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
