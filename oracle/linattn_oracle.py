"""Float64 CPU oracle for SANA's ReLU linear attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
module imports nothing from the product path.

Every function works in float64 on arrays shaped [B, H, N, D] (D innermost) and
follows the pages' definitions step by step, using NumPy's matmul as the only
library primitive.  There is no blocking, fusion or reordering beyond what the
definitions state.

Sources (page title, section):
  [Sana note]   "Sana: Efficient High-Resolution Image Synthesis with Linear
                Diffusion Transformers" (AI-research note, zhao9797.github.io),
                section "Model architecture", item 2) Linear DiT.
  [Video note]  "SANA-Video: Efficient Video Generation with Block Linear
                Diffusion Transformer" (paper notes, shiying-zhang.github.io),
                sections 2.1 (standard linear attention), 2.2 (RoPE
                integration), 2.3 (causal linear attention, constant-memory KV
                cache), 3 Stage 2 (3D RoPE) and 4 (block linear diffusion
                inference algorithm).
  [Video news]  SANA-Video news article (mjgaz.cn), section "Design details"
                (block-causal linear attention and the KV1 -> KV1-2 -> KVsum
                accumulation).

Readings where the pages are silent or garbled (each one is listed with its
reason in the design notes of this repository):
  * eps is added to the denominator after the dot product: d_i = phi(Q_i).z + eps.
    The printed formula of [Video note] 2.1 is lost; the denominator's shape
    follows from the second shared term of [Sana note] item 2).
  * No 1/sqrt(D) scale: the pages mention none.
  * phi = ReLU applies to Q and K only; V is used raw ([Sana note] item 2
    names ReLU(K_j)^T V_j).
  * RoPE pairing is interleaved: pair p rotates dims (2p, 2p+1) by angle theta
    as (x0 cos - x1 sin, x0 sin + x1 cos).  3D split over (t, h, w) is 8/12/12
    dims, base 10000, angle of pair k of an axis of width d_a is
    pos_a * base**(-2k/d_a); token order is n = (t*Hl + h)*Wl + w.  The pages
    say only "3D RoPE" ([Video note] 3 Stage 2), so parity of this convention
    against the pages is unpinned; the tests pin it only to itself through
    invariants (identity angles, shift invariance, norm preservation).
  * Block-causal visibility: a token sees every token of its own chunk and of
    all earlier chunks, never a later chunk ([Video news] "Design details";
    [Video note] 2.3).
  * Projection fused with the state (the QKV projection upstream of the
    attention, [Sana note] "Infra": fusing work into the matmul): the keys and
    values are the per-head projections of the layer input, K = x W_k and
    V = x W_v, each rounded to bfloat16 as a bf16 projection stores them, and
    the state is kv_state of those.  No bias (the pages show none).
  * Backward: the pages say the linear attention's forward and backward passes
    are fused kernels ([Sana note] "Infra") and that the block-causal model is
    trained ([Video note] 3), but print no gradient formulas.  The gradients
    here are those of L = sum_i dout_i . O_i, by the chain rule through the
    forward above, with ReLU'(0) = 0 (the subgradient that keeps exact-zero
    inputs out of the gradient).
"""

import numpy as np


# --------------------------------------------------------------------------
# Feature map and rotation
# --------------------------------------------------------------------------

def feature_map(x):
    """phi = ReLU, the kernel feature map of the linear attention.

    [Sana note] item 2): vanilla softmax self-attention is replaced by ReLU
    linear attention.  max(x, 0) maps -0.0 to +0.0 like the kernels' integer max.
    """
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0)


def rope3d_angles(T, Hl, Wl, D=32, split=(8, 12, 12), base=10000.0):
    """Rotation angles theta[n, p] (float64) of the 3D RoPE, shape [T*Hl*Wl, D/2].

    [Video note] 3 Stage 2 extends rotary position encoding to space-time; the
    per-axis split, base and pairing are this repository's stated reading.
    Axis a (t, h, w) owns split[a] consecutive dims, i.e. split[a]/2 pairs; pair
    k of axis a at coordinate c gets angle c * base**(-2k/split[a]).
    """
    if sum(split) != D or any(s % 2 for s in split):
        raise ValueError("split must be even widths summing to D")
    t = np.arange(T, dtype=np.float64)
    h = np.arange(Hl, dtype=np.float64)
    w = np.arange(Wl, dtype=np.float64)
    tt, hh, ww = np.meshgrid(t, h, w, indexing="ij")     # token n = (t*Hl + h)*Wl + w
    coords = [tt.reshape(-1), hh.reshape(-1), ww.reshape(-1)]
    cols = []
    for axis, width in enumerate(split):
        k = np.arange(width // 2, dtype=np.float64)
        freq = base ** (-2.0 * k / width)
        cols.append(coords[axis][:, None] * freq[None, :])
    return np.concatenate(cols, axis=1)


def rotate_pairs(x, angles):
    """Rotate interleaved pairs (2p, 2p+1) of x[..., N, D] by angles[N, D/2]."""
    x = np.asarray(x, dtype=np.float64)
    c = np.cos(angles)
    s = np.sin(angles)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _positions(angles, n, pos_offset):
    if angles is None:
        return None
    if pos_offset < 0 or pos_offset + n > angles.shape[0]:
        raise ValueError("positions run past the angle table")
    return angles[pos_offset:pos_offset + n]


# --------------------------------------------------------------------------
# Linear (state) forms
# --------------------------------------------------------------------------

def kv_state(k, v, angles=None, pos_offset=0):
    """Shared terms of one token range: S = sum_j phi~(K_j)^T V_j and z = sum_j phi(K_j).

    [Sana note] item 2): sum ReLU(K_j)^T V_j (D x D) and sum ReLU(K_j) are
    computed once and reused by every query.  [Video note] 2.2: with RoPE the
    numerator state holds the rotated keys R_j phi(K_j); the key sum z stays
    un-rotated because the denominator carries no RoPE.

    Returns S[..., D, D] (row = key feature d, column = value feature e) and
    z[..., D].
    """
    phik = feature_map(k)
    v = np.asarray(v, dtype=np.float64)
    pos = _positions(angles, phik.shape[-2], pos_offset)
    phik_num = phik if pos is None else rotate_pairs(phik, pos)
    S = np.matmul(np.swapaxes(phik_num, -1, -2), v)
    z = phik.sum(axis=-2)
    return S, z


def apply_state(q, S, z, eps, angles=None, pos_offset=0):
    """O_i = phi~(Q_i).S / (phi(Q_i).z + eps).

    [Video note] 2.1: once the shared sum is precomputed each token costs
    O(D^2).  [Video note] 2.2: RoPE (if any) rotates phi(Q_i) in the numerator
    only; the denominator uses the un-rotated phi(Q_i) and z.
    """
    phiq = feature_map(q)
    pos = _positions(angles, phiq.shape[-2], pos_offset)
    phiq_num = phiq if pos is None else rotate_pairs(phiq, pos)
    num = np.matmul(phiq_num, S)
    den = np.matmul(phiq, z[..., :, None]) + eps
    return num / den


def linattn(q, k, v, eps=1e-6, angles=None):
    """Non-causal ReLU linear attention over the whole sequence (positions 0..N-1)."""
    S, z = kv_state(k, v, angles)
    return apply_state(q, S, z, eps, angles)


def state_update(k, v, S, z, angles=None, pos_offset=0):
    """Commit one token range into a carried state: (S + S_range, z + z_range).

    [Video note] 2.3 and 4: the constant-memory cache holds the running sums
    of S_j = phi(K_j)^T V_j and of phi(K_j); [Video news] "Design details":
    KV1 + KV2 -> KV1-2 ... -> KVsum.
    """
    dS, dz = kv_state(k, v, angles, pos_offset)
    return np.asarray(S, dtype=np.float64) + dS, np.asarray(z, dtype=np.float64) + dz


def block_forward(q, k, v, S_in, z_in, eps=1e-6, angles=None, pos_offset=0):
    """One chunk of block-causal attention: the chunk's queries see the carried
    state of earlier chunks plus the whole chunk itself.

    [Video news] "Design details": each block's work is the sum of KVsum (the
    earlier blocks) and the block's own KV.  Returns (O_chunk, S_new, z_new);
    S_new/z_new is what a commit stores.
    """
    S_new, z_new = state_update(k, v, S_in, z_in, angles, pos_offset)
    o = apply_state(q, S_new, z_new, eps, angles, pos_offset)
    return o, S_new, z_new


def block_causal(q, k, v, chunk, eps=1e-6, angles=None):
    """Block-causal attention over a whole sequence split into chunks of `chunk`
    tokens (the last one may be shorter), carrying (S, z) from chunk to chunk
    as the recurrence S_c = S_{c-1} + KV_c of [Video note] 2.3.

    Returns (O, S_final, z_final).
    """
    q = np.asarray(q, dtype=np.float64)
    N, D = q.shape[-2], q.shape[-1]
    lead = q.shape[:-2]
    S = np.zeros(lead + (D, D))
    z = np.zeros(lead + (D,))
    out = np.empty(q.shape)
    for start in range(0, N, chunk):
        sl = slice(start, min(N, start + chunk))
        o, S, z = block_forward(q[..., sl, :], k[..., sl, :], v[..., sl, :], S, z,
                                eps, angles, start)
        out[..., sl, :] = o
    return out, S, z


# --------------------------------------------------------------------------
# Quadratic (brute-force) forms
# --------------------------------------------------------------------------

def brute_force(q, k, v, eps=1e-6, angles=None, chunk=None):
    """Softmax-free quadratic attention, O(N^2 D): the definition the linear form
    reaches by associativity ([Video news] "Design details": decomposing along
    the token sequence is mathematically equivalent to the full pairwise form;
    [Video note] 2.1).

    A_ij = phi(Q_i).phi(K_j)          (denominator weights, never rotated)
    A'_ij = (R_i phi(Q_i)).(R_j phi(K_j))  (numerator weights; = A_ij without RoPE)
    M_ij = [chunk(j) <= chunk(i)] in block-causal mode, else 1.
    O_i = sum_j M_ij A'_ij V_j / (sum_j M_ij A_ij + eps)
    """
    phiq = feature_map(q)
    phik = feature_map(k)
    v = np.asarray(v, dtype=np.float64)
    N = phiq.shape[-2]
    A = np.matmul(phiq, np.swapaxes(phik, -1, -2))
    if angles is None:
        A_num = A
    else:
        pos = _positions(angles, N, 0)
        A_num = np.matmul(rotate_pairs(phiq, pos), np.swapaxes(rotate_pairs(phik, pos), -1, -2))
    if chunk is not None:
        idx = np.arange(N) // chunk
        M = (idx[None, :] <= idx[:, None]).astype(np.float64)
        A = A * M
        A_num = A_num * M
    return np.matmul(A_num, v) / (A.sum(axis=-1, keepdims=True) + eps)


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

def backward(q, k, v, dout, eps=1e-6, angles=None, chunk=None, S_in=None, z_in=None, dS_out=None, dz_out=None):
    """Gradients of L = sum_i dout_i . O_i (+ <dS_out, S_out> + dz_out . z_out)
    for block-causal attention with chunks of `chunk` tokens (None: one chunk,
    i.e. non-causal) started from the carried state (S_in, z_in), where
    (S_out, z_out) is the state after the last chunk (what a commit stores).

    The forward of [Video note] 2.1-2.3 per chunk c, with S_c = S_in + the
    chunks up to and including c (and z_c likewise):
      num_i = phi~(Q_i) S_c,  den_i = phi(Q_i).z_c + eps,  O_i = num_i / den_i.
    Chain rule, query side (tokens i of chunk c):
      dnum_i = dout_i / den_i,  dden_i = -(dout_i . num_i) / den_i^2
      dphi(Q_i) = R_i^T (S_c dnum_i) + z_c dden_i,  dQ_i = [Q_i > 0] dphi(Q_i)
      dS_c = sum_i phi~(Q_i) dnum_i^T,  dz_c = sum_i phi(Q_i) dden_i.
    Key side: chunk c's keys enter every S_c' with c' >= c and S_out, so with
      G_c = dS_out + sum_{c' >= c} dS_c'  (Gz_c likewise)
      dphi(K_j) = R_j^T (G_c V_j) + Gz_c,  dK_j = [K_j > 0] dphi(K_j),
      dV_j = G_c^T phi~(K_j).
    The carried state enters every S_c and S_out: dS_in = G_0, dz_in = Gz_0.

    Returns (dq, dk, dv, dS_in, dz_in).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    N, D = q.shape[-2], q.shape[-1]
    lead = q.shape[:-2]
    L = N if chunk is None else chunk
    phiq = feature_map(q)
    phik = feature_map(k)
    pos = _positions(angles, N, 0)
    phiq_num = phiq if pos is None else rotate_pairs(phiq, pos)
    phik_num = phik if pos is None else rotate_pairs(phik, pos)
    chunks = [slice(start, min(N, start + L)) for start in range(0, N, L)]

    # forward states: S_c, z_c after each chunk
    S = np.zeros(lead + (D, D)) if S_in is None else np.asarray(S_in, dtype=np.float64)
    z = np.zeros(lead + (D,)) if z_in is None else np.asarray(z_in, dtype=np.float64)
    states = []
    for sl in chunks:
        S = S + np.matmul(np.swapaxes(phik_num[..., sl, :], -1, -2), v[..., sl, :])
        z = z + phik[..., sl, :].sum(axis=-2)
        states.append((S, z))

    # query side
    dq = np.zeros(q.shape)
    dS_chunk, dz_chunk = [], []
    for sl, (S_c, z_c) in zip(chunks, states):
        num = np.matmul(phiq_num[..., sl, :], S_c)
        den = np.matmul(phiq[..., sl, :], z_c[..., :, None]) + eps
        dnum = dout[..., sl, :] / den
        dden = -(dout[..., sl, :] * num).sum(axis=-1, keepdims=True) / den ** 2
        dphiq_num = np.matmul(dnum, np.swapaxes(S_c, -1, -2))
        dphiq_rot = dphiq_num if pos is None else rotate_pairs(dphiq_num, -pos[sl])
        dphiq = dphiq_rot + dden * z_c[..., None, :]
        dq[..., sl, :] = dphiq * (q[..., sl, :] > 0)
        dS_chunk.append(np.matmul(np.swapaxes(phiq_num[..., sl, :], -1, -2), dnum))
        dz_chunk.append((phiq[..., sl, :] * dden).sum(axis=-2))

    # key side: suffix sums of the query-side state gradients
    G = np.zeros(lead + (D, D)) if dS_out is None else np.asarray(dS_out, dtype=np.float64)
    Gz = np.zeros(lead + (D,)) if dz_out is None else np.asarray(dz_out, dtype=np.float64)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for c in range(len(chunks) - 1, -1, -1):
        sl = chunks[c]
        G = G + dS_chunk[c]
        Gz = Gz + dz_chunk[c]
        dphik_num = np.matmul(v[..., sl, :], np.swapaxes(G, -1, -2))
        dphik_rot = dphik_num if pos is None else rotate_pairs(dphik_num, -pos[sl])
        dphik = dphik_rot + Gz[..., None, :]
        dk[..., sl, :] = dphik * (k[..., sl, :] > 0)
        dv[..., sl, :] = np.matmul(phik_num[..., sl, :], G)
    return dq, dk, dv, G, Gz


# --------------------------------------------------------------------------
# Temporal convolution of the block-inference cache
# --------------------------------------------------------------------------

def temporal_conv3(x, w, bias=None, prev_frame=None):
    """Shortcut-integrated temporal convolution over frames, block-causal:
    y[b, f, s, c] = x[b, f, s, c] + w[c, 0] x[b, f-1, s, c] + w[c, 1] x[b, f, s, c]
                    + w[c, 2] x[b, f+1, s, c] + bias[c]
    with x[b, -1] = prev_frame[b] (zeros when None) and x[b, F] = 0.

    [Video news] "Design details": the Spatial-Temporal Mix-FFN uses 3x1x1
    temporal filters; [Video note] 3 Stage 2: the 1D temporal convolution enters
    the Mix-FFN through a shortcut; [Video note] 4: the block-inference cache
    keeps the conv's last frame.  Readings: depthwise (one filter per channel,
    as the Mix-FFN's spatial conv is depth-wise); the previous chunk's last
    frame is the only context across a chunk boundary, and a chunk sees no
    later frame (zero padding at its end).

    x: [B, F, S, C] (frames, spatial tokens, channels); w: [C, 3]; bias: [C];
    prev_frame: [B, S, C].  Returns y [B, F, S, C] and the cache for the next
    chunk, x[:, F-1].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, F, S, C = x.shape
    prev = np.zeros((B, S, C)) if prev_frame is None else np.asarray(prev_frame, dtype=np.float64)
    padded = np.concatenate([prev[:, None], x, np.zeros((B, 1, S, C))], axis=1)
    y = x + w[:, 0] * padded[:, :F] + w[:, 1] * padded[:, 1:F + 1] + w[:, 2] * padded[:, 2:F + 2]
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y, x[:, F - 1].copy()


# --------------------------------------------------------------------------
# The key/value projection feeding the state
# --------------------------------------------------------------------------

def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (8 significant bits,
    ties to even), for values in bfloat16's normal range and zero."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def projected_kv_state(x, w_k, w_v, angles=None, pos_offset=0):
    """State of the keys and values a layer's projection produces.

    x: [B, N, C] layer input; w_k, w_v: [H, C, D] per-head projection weights.
    K[b, h] = x[b] W_k[h] and V[b, h] = x[b] W_v[h] (float64 products and
    sums), each rounded to bfloat16 as the projection output is stored, then
    S = sum_n phi~(K_n)^T V_n and z = sum_n phi(K_n) per (batch, head), as in
    kv_state ([Sana note] item 2); [Sana note] "Infra" for the fusion with the
    matmul).  With angles, key n of every batch is rotated at position
    pos_offset + n after the ReLU, in S only ([Video note] 2.2).  Returns
    S [B, H, D, D], z [B, H, D].
    """
    x = np.asarray(x, dtype=np.float64)[:, None]          # [B, 1, N, C]
    k = round_bf16(np.matmul(x, np.asarray(w_k, dtype=np.float64)[None]))
    v = round_bf16(np.matmul(x, np.asarray(w_v, dtype=np.float64)[None]))
    return kv_state(k, v, angles, pos_offset)


def projected_apply(x, w_q, S, z, eps, angles=None, pos_offset=0):
    """Outputs of the queries a layer's projection produces, against a given
    state.

    x: [B, N, C] layer input; w_q: [H, C, D] per-head query weights; S
    [B, H, D, D], z [B, H, D]: the state (for example projected_kv_state's).
    Q[b, h] = x[b] W_q[h] (float64), rounded to bfloat16 as the projection
    output is stored, then O = phi~(Q).S / (phi(Q).z + eps) as in apply_state
    ([Video note] 2.1, 2.2; [Sana note] "Infra" for the fusion with the
    matmul).  Returns O [B, H, N, D].
    """
    x = np.asarray(x, dtype=np.float64)[:, None]          # [B, 1, N, C]
    q = round_bf16(np.matmul(x, np.asarray(w_q, dtype=np.float64)[None]))
    return apply_state(q, np.asarray(S, dtype=np.float64), np.asarray(z, dtype=np.float64), eps, angles, pos_offset)
