// Backward kernels of SANA's ReLU linear attention (gfx950).
//
// For L = sum_i dO_i . O_i (+ the gradient reaching the committed state), with
// chunk c's state S_c = S_in + chunks 0..c (z_c likewise), the chain rule
// through the forward gives, per query i of chunk c,
//   den_i = phi(Q_i).z_c + eps,  num_i = phi~(Q_i).S_c
//   dnum_i = dO_i / den_i,  dden_i = -(dO_i . num_i) / den_i^2
//   dQ_i = [Q_i > 0] (R_i^T (S_c dnum_i) + z_c dden_i)
//   dS_c = sum_i phi~(Q_i) dnum_i^T,  dz_c = sum_i phi(Q_i) dden_i
// and, with the suffix sums G_c = dS_out + sum_{c' >= c} dS_c' (Gz_c likewise),
// per key j of chunk c,
//   dK_j = [K_j > 0] (R_j^T (G_c V_j) + Gz_c),  dV_j = G_c^T phi~(K_j)
// and dS_in = G_0.  "Sana" research note, Infra: the linear attention's
// forward and backward are fused kernels; "SANA-Video" paper notes 3: the
// block-causal model is trained.  ReLU'(0) is taken as 0.
//
// Pipeline (host side): the forward state pass and finalize recompute S_c;
// bwd_query computes dQ and one partial (dS, dz) per workgroup; the reverse
// finalize walks each head's partials from the last chunk to the first,
// storing G_c at every chunk start; bwd_key computes dK and dV.
//
// The *_vec kernels keep the arithmetic in fp32 on the VALU (fp32 I/O); the
// bf16 kernels put the contractions on v_mfma_f32_16x16x32_bf16 with the same
// exact three-part splits of fp32 operands as the forward.
#pragma once

#include "la_kernels.h"

namespace la {

// ---------------------------------------------------------------------------
// fp32 element I/O: four consecutive features
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4_t load4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }

__device__ __forceinline__ void store4(float* p, f32x4_t x) { *reinterpret_cast<f32x4_t*>(p) = x; }

// Sum over the 8 consecutive lanes that share a token
__device__ __forceinline__ float sum8(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

// Features f0 .. f0+3 (two pairs) of the token at position pos rotated by
// +theta (forward) or -theta (the transpose, on the way back).
template <bool INVERSE, int ROPE>
__device__ __forceinline__ f32x4_t rotate4(f32x4_t x, const Rope& rp, const float* rtab, int64_t pos, int f0) {
  f32x4_t y;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float c, s;
    rope_pair<ROPE>(rp, rtab, pos, f0 / 2 + u, c, s);
    if (INVERSE) s = -s;
    y[2 * u] = rot_lo(x[2 * u], x[2 * u + 1], c, s);
    y[2 * u + 1] = rot_hi(x[2 * u], x[2 * u + 1], c, s);
  }
  return y;
}

// ---------------------------------------------------------------------------
// Reverse finalize: suffix sums of the query pass's partial state gradients
// ---------------------------------------------------------------------------
//
// One thread per state element of every head.  It starts from the gradient
// reaching the committed state (kv_in/ksum_in of `a`, or 0), walks the head's
// C x Pc partials from the last to the first, BATCH loads in flight at a time
// (issued unconditionally, as in state_finalize), stores the running sum at
// the start of every chunk (G_c) and commits the total (G_0, the gradient of
// the carried state) to kv_out/ksum_out.
template <int BATCH>
__global__ __launch_bounds__(kThreads) void state_finalize_reverse(StateArgs a, int64_t n_elems) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_elems) return;
  const int64_t bh = i / kStateElems;
  const int idx = (int)(i % kStateElems);
  const int total = a.C * a.Pc;
  const float* src = a.partials + bh * total * kStateElems + idx;
  float* dst = a.states + bh * a.C * kStateElems + idx;
  float acc = carried(a, bh, idx);
  int c = a.C - 1, s = a.Pc - 1;  // chunk and split of the next partial
  for (int q1 = total; q1 > 0; q1 -= BATCH) {
    // slot u holds partial q1 - 1 - u (the first partial again once past it)
    const int nb = q1 < BATCH ? q1 : BATCH;
    float v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) v[u] = src[(int64_t)max(q1 - 1 - u, 0) * kStateElems];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (u < nb) {
        acc += v[u];
        if (s == 0) {
          dst[(int64_t)c * kStateElems] = acc;
          s = a.Pc - 1;
          --c;
        } else {
          --s;
        }
      }
    }
  }
  if (a.kv_out) commit(a, bh, idx, acc);
}

// ---------------------------------------------------------------------------
// Query pass: dQ and the partial (dS, dz) of one token range
// ---------------------------------------------------------------------------
//
// Workgroup = item (head, chunk, split) of the state-pass geometry; it reads
// S_c, z_c through `fwd` and writes its partial through `a` (a.kv_in/ksum_in:
// gradient reaching the committed state, added when the head has a single
// item; a.kv_out/ksum_out: where that case commits dS_in).  32-token tiles:
// thread t handles features f0 = 4 (t % 8) .. f0+3 of token t / 8 of the
// tile, and element row d = t / 8, columns f0 .. f0+3 of the partial dS.
template <int ROPE>
__global__ __launch_bounds__(kThreads) void bwd_query_vec(const float* __restrict__ Q, const float* __restrict__ dO,
                                                          float* __restrict__ dQ, Layout lin, Layout lout,
                                                          StateView fwd, float eps, Rope rp, StateArgs a) {
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  __shared__ float sS[kD][kD + 1];
  __shared__ float sz[kD];
  __shared__ float sp[32][kD + 1];   // phi(Q)
  __shared__ float spr[32][kD + 1];  // phi~(Q)
  __shared__ float sdn[32][kD + 1];  // dnum
  __shared__ float sdd[32];          // dden
  __shared__ float mine[kStateElems];

  int64_t bh, n_begin, n_end;
  int c, s;
  state_item(a, bh, c, s, n_begin, n_end);
  const int t = threadIdx.x;
  const int tl = t >> 3;
  const int f0 = (t & 7) * 4;
  const int64_t sc = bh * a.C + c;
  for (int idx = t; idx < kD * kD; idx += kThreads) sS[idx >> 5][idx & 31] = fwd.s_base[sc * fwd.s_stride + idx];
  if (t < kD) sz[t] = fwd.z_base[sc * fwd.z_stride + t];
  rope_stage<ROPE>(rp, rtab, t, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  for (int64_t t0 = n_begin; t0 < n_end; t0 += 32) {
    const int64_t tok = t0 + tl;
    const bool live = tok < n_end;
    const int64_t row = lin.base(bh) + tok * lin.token + f0;
    f32x4_t x = {0.f, 0.f, 0.f, 0.f}, g = x;
    if (live) {
      x = load4(Q + row);
      g = load4(dO + row);
    }
    f32x4_t p, pr;
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = fmaxf(x[u], 0.f);
    pr = p;
    if constexpr (ROPE) {
      if (live) pr = rotate4<false, ROPE>(p, rp, rtab, rp.pos0 + tok, f0);
    }
    __syncthreads();  // previous tile's readers are done (and S, z are in place)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sp[tl][f0 + u] = p[u];
      spr[tl][f0 + u] = pr[u];
    }
    __syncthreads();
    float den = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) den += p[u] * sz[f0 + u];
    den = sum8(den) + eps;
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
    for (int d = 0; d < kD; ++d) {
      const float qd = spr[tl][d];
#pragma unroll
      for (int u = 0; u < 4; ++u) num[u] += qd * sS[d][f0 + u];
    }
    // rows past the split's end carry zeros: they must add nothing, eps = 0 included
    const float rden = live ? 1.f / den : 0.f;
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sdn[tl][f0 + u] = g[u] * rden;
      dot += g[u] * num[u];
    }
    const float dden = -sum8(dot) * rden * rden;
    if ((t & 7) == 0) sdd[tl] = dden;
    __syncthreads();
    // dQ for features f0 .. f0+3 of this token
    f32x4_t dr = {0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < kD; ++e) {
      const float de = sdn[tl][e];
#pragma unroll
      for (int u = 0; u < 4; ++u) dr[u] += sS[f0 + u][e] * de;
    }
    if constexpr (ROPE) {
      if (live) dr = rotate4<true, ROPE>(dr, rp, rtab, rp.pos0 + tok, f0);
    }
    f32x4_t dq;
#pragma unroll
    for (int u = 0; u < 4; ++u) dq[u] = x[u] > 0.f ? dr[u] + sz[f0 + u] * dden : 0.f;
    if (live) store4(dQ + lout.base(bh) + tok * lout.token + f0, dq);
    // partial dS row d = tl, columns f0 .. f0+3; dz[d]
    for (int j = 0; j < 32; ++j) {
      const float qd = spr[j][tl];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += qd * sdn[j][f0 + u];
      zacc += sp[j][tl] * sdd[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) mine[tl * 32 + f0 + u] = acc[u];
  if (f0 == 0) mine[1024 + tl] = zacc;
  __syncthreads();
  write_partial(mine, bh, c, s, a);
}

// ---------------------------------------------------------------------------
// Key pass: dK and dV from G_c
// ---------------------------------------------------------------------------
//
// Workgroup (head, chunk, tile) takes tokens [c*L + tile*Lt, ...) of chunk c;
// 32-token tiles, thread t: features f0 = 4 (t % 8) .. f0+3 of token t / 8.
template <int ROPE>
__global__ __launch_bounds__(kThreads) void bwd_key_vec(const float* __restrict__ K, const float* __restrict__ V,
                                                        float* __restrict__ dK, float* __restrict__ dV, Layout lin,
                                                        Layout lout, StateView grad,
                                                        int64_t N, int64_t L, int C, int tiles, int64_t Lt,
                                                        Rope rp) {
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  __shared__ float sG[kD][kD + 1];
  __shared__ float sGz[kD];
  __shared__ float skr[32][kD + 1];  // phi~(K)
  __shared__ float sv[32][kD + 1];

  const int64_t bh = blockIdx.x / ((int64_t)C * tiles);
  const int r = (int)(blockIdx.x % ((int64_t)C * tiles));
  const int c = r / tiles;
  const int tile = r % tiles;
  const int64_t c_end = ((int64_t)c + 1) * L < N ? ((int64_t)c + 1) * L : N;
  const int64_t n_begin = (int64_t)c * L + (int64_t)tile * Lt;
  const int64_t n_end = (n_begin + Lt < c_end) ? n_begin + Lt : c_end;
  const int t = threadIdx.x;
  const int tl = t >> 3;
  const int f0 = (t & 7) * 4;
  const int64_t sc = bh * C + c;
  for (int idx = t; idx < kD * kD; idx += kThreads) sG[idx >> 5][idx & 31] = grad.s_base[sc * grad.s_stride + idx];
  if (t < kD) sGz[t] = grad.z_base[sc * grad.z_stride + t];
  rope_stage<ROPE>(rp, rtab, t, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  for (int64_t t0 = n_begin; t0 < n_end; t0 += 32) {
    const int64_t tok = t0 + tl;
    const bool live = tok < n_end;
    const int64_t row = lin.base(bh) + tok * lin.token + f0;
    const int64_t orow = lout.base(bh) + tok * lout.token + f0;
    f32x4_t x = {0.f, 0.f, 0.f, 0.f}, vv = x;
    if (live) {
      x = load4(K + row);
      vv = load4(V + row);
    }
    f32x4_t p;
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = fmaxf(x[u], 0.f);
    if constexpr (ROPE) {
      if (live) p = rotate4<false, ROPE>(p, rp, rtab, rp.pos0 + tok, f0);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      skr[tl][f0 + u] = p[u];
      sv[tl][f0 + u] = vv[u];
    }
    __syncthreads();
    f32x4_t dv = {0.f, 0.f, 0.f, 0.f}, dr = dv;
    for (int j = 0; j < kD; ++j) {
      const float kj = skr[tl][j];  // key feature d = j
      const float vj = sv[tl][j];   // value feature e = j
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dv[u] += sG[j][f0 + u] * kj;
        dr[u] += sG[f0 + u][j] * vj;
      }
    }
    if constexpr (ROPE) {
      if (live) dr = rotate4<true, ROPE>(dr, rp, rtab, rp.pos0 + tok, f0);
    }
    f32x4_t dk;
#pragma unroll
    for (int u = 0; u < 4; ++u) dk[u] = x[u] > 0.f ? dr[u] + sGz[f0 + u] : 0.f;
    if (live) {
      store4(dK + orow, dk);
      store4(dV + orow, dv);
    }
  }
}

// ===========================================================================
// bf16 kernels (MFMA)
// ===========================================================================
//
// Natural layout as in the apply pass: lane l (m = l % 16, g = l / 16) holds
// features 8g .. 8g+7 of token row m of a 16-token tile, and MFMA output half
// h row r stands for feature 8(r / 4) + 4h + r % 4, so each lane ends with the
// outputs of its own 8 features.

// A operand whose rows are the rows r of a 32 x 32 fp32 matrix M (row of MFMA
// half h = 8(m / 4) + 4h + m % 4) and whose k-slot s of group g is column
// 8g + s: M[r][8g + s] in three bf16 parts.  Against B = X^T (k = column
// index, one column per token) it gives (M x)[r] per token.
__device__ __forceinline__ void load_row_operands(const float* M, int g, int m, bf16x8_t (&a)[2][3]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * (m >> 2) + 4 * h + (m & 3);
    unsigned part[3][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      split3_bf16x2(M[r * 32 + 8 * g + 2 * p], M[r * 32 + 8 * g + 2 * p + 1], part[0][p], part[1][p], part[2][p]);
#pragma unroll
    for (int k = 0; k < 3; ++k) a[h][k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
  }
}

// A operand whose rows are the columns e of M (M^T, same row mapping) and
// whose k-slot s of group g is row 8g + s: M[8g + s][e].  Gives (M^T x)[e].
__device__ __forceinline__ void load_column_operands(const float* M, int g, int m, bf16x8_t (&a)[2][3]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 8 * (m >> 2) + 4 * h + (m & 3);
    unsigned part[3][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      split3_bf16x2(M[(8 * g + 2 * p) * 32 + e], M[(8 * g + 2 * p + 1) * 32 + e], part[0][p], part[1][p],
                    part[2][p]);
#pragma unroll
    for (int k = 0; k < 3; ++k) a[h][k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
  }
}

// A vector v[32] broadcast to every row: k-slot s of group g holds v[8g + s].
__device__ __forceinline__ void load_vector_operands(const float* v, int g, bf16x8_t (&a)[3]) {
  unsigned part[3][4];
#pragma unroll
  for (int p = 0; p < 4; ++p) split3_bf16x2(v[8 * g + 2 * p], v[8 * g + 2 * p + 1], part[0][p], part[1][p], part[2][p]);
#pragma unroll
  for (int k = 0; k < 3; ++k) a[k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
}

// Split operand a (three parts) times an exact bf16 operand b, both halves
__device__ __forceinline__ void mfma3(const bf16x8_t (&a)[2][3], bf16x8_t b, f32x4_t& o0, f32x4_t& o1) {
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  o0 = mfma16(a[0][0], b, zero4);
  o0 = mfma16(a[0][1], b, o0);
  o0 = mfma16(a[0][2], b, o0);
  o1 = mfma16(a[1][0], b, zero4);
  o1 = mfma16(a[1][1], b, o1);
  o1 = mfma16(a[1][2], b, o1);
}

// Two split operands: the six product terms of weight >= 2^-16
__device__ __forceinline__ void mfma6(const bf16x8_t (&a)[2][3], const bf16x8_t (&b)[3], f32x4_t& o0,
                                      f32x4_t& o1) {
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t* o[2] = {&o0, &o1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4_t x = mfma16(a[h][0], b[0], zero4);
    x = mfma16(a[h][0], b[1], x);
    x = mfma16(a[h][1], b[0], x);
    x = mfma16(a[h][0], b[2], x);
    x = mfma16(a[h][2], b[0], x);
    x = mfma16(a[h][1], b[1], x);
    *o[h] = x;
  }
}

__device__ __forceinline__ void unpack8(u32x4_t x, float (&f)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f[2 * p] = bf16lo_to_f32(x[p]);
    f[2 * p + 1] = bf16hi_to_f32(x[p]);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float (&f)[8]) {
  return u32x4_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// Rotate the lane's 4 pairs (x[2p], x[2p+1]) by +theta (INVERSE: -theta)
template <bool INVERSE>
__device__ __forceinline__ void rotate8(float (&x)[8], f32x4_t c, f32x4_t sn) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float s = INVERSE ? -sn[p] : sn[p];
    const float x0 = x[2 * p], x1 = x[2 * p + 1];
    x[2 * p] = rot_lo(x0, x1, c[p], s);
    x[2 * p + 1] = rot_hi(x0, x1, c[p], s);
  }
}

__device__ __forceinline__ void split8(const float (&y)[8], bf16x8_t (&b)[3]) {
  unsigned part[3][4];
#pragma unroll
  for (int p = 0; p < 4; ++p) split3_bf16x2(y[2 * p], y[2 * p + 1], part[0][p], part[1][p], part[2][p]);
#pragma unroll
  for (int k = 0; k < 3; ++k) b[k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
}

// ---------------------------------------------------------------------------
// Key pass (bf16): per 16-token tile, dV = G^T phi~(K) and
// dK = [K > 0] (R^T (G V) + Gz); both outputs in the natural layout.
// Work split as the apply pass: equal flat ranges cut at head and chunk
// boundaries; each wave takes 64-token chunks (four tiles) with the next
// chunk's loads in flight.
// ---------------------------------------------------------------------------

template <int ROPE>
struct KeyChunk {
  u32x4_t k[4], v[4];
  f32x4_t c[4], sn[4];
};

template <int ROPE>
__device__ __forceinline__ void load_key_chunk(const char* Kh, const char* Vh, int64_t row, int64_t t0,
                                               int64_t n_end, int lane_off, int tab_off, int m, int g,
                                               const Rope& rp, const float* rtab, const AxisLane& al,
                                               KeyChunk<ROPE>& ch) {
  const rsrc_t rk = rows_rsrc(Kh, t0, n_end, row);
  const rsrc_t rv = rows_rsrc(Vh, t0, n_end, row);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ch.k[u] = load16_nt(rk, lane_off + u * 16 * (int)row);
    ch.v[u] = load16_nt(rv, lane_off + u * 16 * (int)row);
  }
  if constexpr (ROPE == kRopeTable) {
    const rsrc_t rc = make_rsrc(rp.cos + (rp.pos0 + t0) * 16, (n_end - t0) * 64);
    const rsrc_t rs = make_rsrc(rp.sin + (rp.pos0 + t0) * 16, (n_end - t0) * 64);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ch.c[u] = load16(rc, tab_off + u * 1024);
      ch.sn[u] = load16(rs, tab_off + u * 1024);
    }
  }
  // the axis form's angles come from LDS when the tile is computed
}

template <int ROPE, bool DENSE>
__global__ __launch_bounds__(kThreads) void bwd_key_bf16(const u32x4_t* __restrict__ K, const u32x4_t* __restrict__ V,
                                                         u32x4_t* __restrict__ dK, u32x4_t* __restrict__ dV,
                                                         Layout lin, Layout lout, StateView grad, int64_t N,
                                                         int64_t L, int C, int64_t total, int64_t La, Rope rp) {
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only
  const int64_t irow = DENSE ? 64 : lin.token * 2, orow = DENSE ? 64 : lout.token * 2;  // bytes between tokens
  const int lane_off = m * (int)irow + g * 16;
  const int out_off = m * (int)orow + g * 16;
  const int tab_off = m * 64 + g * 16;
  const int64_t f_begin = (int64_t)blockIdx.x * La;
  const int64_t f_end = (f_begin + La < total) ? f_begin + La : total;

  for (int64_t f = f_begin; f < f_end;) {
    const int64_t bh = f / N;
    const int64_t n_begin = f - bh * N;
    const int c = (int)(n_begin / L);
    const int64_t c_end = ((int64_t)c + 1) * L < N ? ((int64_t)c + 1) * L : N;
    const int64_t n_end = (f_end - bh * N < c_end) ? f_end - bh * N : c_end;
    f = bh * N + n_end;
    const char* Kh = reinterpret_cast<const char*>(K) + lin.base(bh) * 2;
    const char* Vh = reinterpret_cast<const char*>(V) + lin.base(bh) * 2;
    char* dKh = reinterpret_cast<char*>(dK) + lout.base(bh) * 2;
    char* dVh = reinterpret_cast<char*>(dV) + lout.base(bh) * 2;

    int64_t t0 = n_begin + 64 * w;
    KeyChunk<ROPE> next;
    if (t0 < n_end) load_key_chunk<ROPE>(Kh, Vh, irow, t0, n_end, lane_off, tab_off, m, g, rp, rtab, al, next);
    const int64_t sc = bh * C + c;
    const float* G = grad.s_base + sc * grad.s_stride;
    const float* Gz = grad.z_base + sc * grad.z_stride;
    bf16x8_t gcol[2][3], grow[2][3];
    load_column_operands(G, g, m, gcol);  // dV = G^T phi~(K)
    load_row_operands(G, g, m, grow);     // G V
    float gz[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) gz[j] = Gz[8 * g + j];

    for (; t0 < n_end; t0 += 256) {
      const KeyChunk<ROPE> cur = next;
      if (t0 + 256 < n_end)
        load_key_chunk<ROPE>(Kh, Vh, irow, t0 + 256, n_end, lane_off, tab_off, m, g, rp, rtab, al, next);
      const rsrc_t rdk = rows_rsrc(dKh, t0, n_end, orow);
      const rsrc_t rdv = rows_rsrc(dVh, t0, n_end, orow);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4_t kr = relu_bf16x8(cur.k[u]);
        f32x4_t o0, o1;
        float x[8];
        f32x4_t ang_c = cur.c[u], ang_s = cur.sn[u];
        if constexpr (ROPE == kRopeAxes) rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 16 * u + m, ang_c, ang_s);
        if constexpr (!ROPE) {
          mfma3(gcol, __builtin_bit_cast(bf16x8_t, kr), o0, o1);
        } else {
          float y[8];
          unpack8(kr, y);
          rotate8<false>(y, ang_c, ang_s);
          bf16x8_t b[3];
          split8(y, b);
          mfma6(gcol, b, o0, o1);
        }
        x[0] = o0[0], x[1] = o0[1], x[2] = o0[2], x[3] = o0[3];
        x[4] = o1[0], x[5] = o1[1], x[6] = o1[2], x[7] = o1[3];
        store16_nt(rdv, out_off + u * 16 * (int)orow, pack8(x));
        mfma3(grow, __builtin_bit_cast(bf16x8_t, cur.v[u]), o0, o1);
        x[0] = o0[0], x[1] = o0[1], x[2] = o0[2], x[3] = o0[3];
        x[4] = o1[0], x[5] = o1[1], x[6] = o1[2], x[7] = o1[3];
        if constexpr (ROPE) rotate8<true>(x, ang_c, ang_s);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          x[2 * p] = (kr[p] & 0xffffu) ? x[2 * p] + gz[2 * p] : 0.f;
          x[2 * p + 1] = (kr[p] >> 16) ? x[2 * p + 1] + gz[2 * p + 1] : 0.f;
        }
        store16_nt(rdk, out_off + u * 16 * (int)orow, pack8(x));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Query pass (bf16): dQ and one partial (dS, dz) per workgroup
// ---------------------------------------------------------------------------
//
// Workgroup = item (head, chunk, split) of the state-pass geometry; each wave
// takes 32-token tiles (two 16-token halves, the next tile's loads in flight).
// Per half, in the natural layout:
//   den (A rows = z), num = S^T phi~(Q) (A = S columns), S dO (A = S rows;
//   dO is exact in bf16, so S dnum = (S dO) / den), dnum = dO / den,
//   dden = -(dO . num) / den^2 (the lane's 8 features, then the 4 lanes of the
//   token), dQ, and dz += phi(Q) dden per feature.
// dS = sum phi~(Q) dnum^T contracts over tokens: dnum (and, under RoPE, the
// rotated phi~(Q)) go through a wave-private LDS tile into the turned-around
// layout (lane (n, g): feature n of tokens 4g + i), phi(Q) without RoPE is
// turned around exactly on the matrix core, and dS accumulates in the
// state pass's layout.
constexpr int kTileRow = 36;                  // padded fp32 row of a 32-feature token
constexpr int kTileFloats = 32 * kTileRow;    // one 32-token tile

template <int ROPE>
struct QueryTile {
  u32x4_t q[2], dout[2];
  f32x4_t c[2], sn[2];
};

template <int ROPE>
__device__ __forceinline__ void load_query_tile(const char* Qh, const char* Oh, int64_t row, int64_t t0,
                                                int64_t n_end, int lane_off, int tab_off, int m, int g,
                                                const Rope& rp, const float* rtab, const AxisLane& al,
                                                QueryTile<ROPE>& tl) {
  const rsrc_t rq = rows_rsrc(Qh, t0, n_end, row);
  const rsrc_t ro = rows_rsrc(Oh, t0, n_end, row);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    tl.q[tb] = load16_nt(rq, lane_off + tb * 16 * (int)row);
    tl.dout[tb] = load16_nt(ro, lane_off + tb * 16 * (int)row);
  }
  if constexpr (ROPE == kRopeTable) {
    const rsrc_t rc = make_rsrc(rp.cos + (rp.pos0 + t0) * 16, (n_end - t0) * 64);
    const rsrc_t rs = make_rsrc(rp.sin + (rp.pos0 + t0) * 16, (n_end - t0) * 64);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      tl.c[tb] = load16(rc, tab_off + tb * 1024);
      tl.sn[tb] = load16(rs, tab_off + tb * 1024);
    }
  }
  // the axis form's angles come from LDS when the tile is computed
}

template <int ROPE, bool DENSE>
__global__ __launch_bounds__(kThreads) void bwd_query_bf16(const u32x4_t* __restrict__ Q,
                                                           const u32x4_t* __restrict__ dO, u32x4_t* __restrict__ dQ,
                                                           Layout lin, Layout lout, StateView fwd, float eps,
                                                           Rope rp, StateArgs a) {
  __shared__ float red[4][kStateElems];
  __shared__ float tiles[4][ROPE ? 2 : 1][kTileFloats];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  int64_t bh, n_begin, n_end;
  int c, s;
  state_item(a, bh, c, s, n_begin, n_end);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;  // also the token row m of the natural layout
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only
  const int64_t irow = DENSE ? 64 : lin.token * 2, orow = DENSE ? 64 : lout.token * 2;  // bytes between tokens
  const int lane_off = n * (int)irow + g * 16;
  const int out_off = n * (int)orow + g * 16;
  const int tab_off = n * 64 + g * 16;
  const char* Qh = reinterpret_cast<const char*>(Q) + lin.base(bh) * 2;
  const char* Oh = reinterpret_cast<const char*>(dO) + lin.base(bh) * 2;
  char* dQh = reinterpret_cast<char*>(dQ) + lout.base(bh) * 2;
  float* dn_tile = tiles[w][0];
  float* pq_tile = tiles[w][ROPE ? 1 : 0];

  int64_t t0 = n_begin + 32 * w;
  QueryTile<ROPE> next;
  if (t0 < n_end) load_query_tile<ROPE>(Qh, Oh, irow, t0, n_end, lane_off, tab_off, n, g, rp, rtab, al, next);

  const int64_t sc = bh * a.C + c;
  const float* S = fwd.s_base + sc * fwd.s_stride;
  const float* Z = fwd.z_base + sc * fwd.z_stride;
  bf16x8_t scol[2][3], srow[2][3], zrow[3];
  load_column_operands(S, g, n, scol);  // num = S^T phi~(Q)
  load_row_operands(S, g, n, srow);     // S dO
  load_vector_operands(Z, g, zrow);     // den
  float zf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zf[j] = Z[8 * g + j];
  const bf16x8_t sel[2] = {select_operand(g, n, 0), select_operand(g, n, 1)};

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float dzacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) dzacc[j] = 0.f;

  for (; t0 < n_end; t0 += 128) {
    const QueryTile<ROPE> cur = next;
    if (t0 + 128 < n_end)
      load_query_tile<ROPE>(Qh, Oh, irow, t0 + 128, n_end, lane_off, tab_off, n, g, rp, rtab, al, next);
    const rsrc_t rdq = rows_rsrc(dQh, t0, n_end, orow);
    bf16x8_t bq[2];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const u32x4_t qr = relu_bf16x8(cur.q[tb]);
      bq[tb] = __builtin_bit_cast(bf16x8_t, qr);
      f32x4_t ang_c = cur.c[tb], ang_s = cur.sn[tb];
      if constexpr (ROPE == kRopeAxes) rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 16 * tb + n, ang_c, ang_s);
      const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
      f32x4_t dacc = mfma16(zrow[0], bq[tb], zero4);
      dacc = mfma16(zrow[1], bq[tb], dacc);
      dacc = mfma16(zrow[2], bq[tb], dacc);
      // rows past the split's end carry zeros: they must add nothing, eps = 0 included
      const float rden = t0 + 16 * tb + n < n_end ? 1.f / (dacc[0] + eps) : 0.f;
      float pq[8], y[8];
      unpack8(qr, pq);
      f32x4_t n0, n1;
      if constexpr (!ROPE) {
        mfma3(scol, bq[tb], n0, n1);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = pq[j];
        rotate8<false>(y, ang_c, ang_s);
        bf16x8_t br[3];
        split8(y, br);
        mfma6(scol, br, n0, n1);
      }
      f32x4_t s0, s1;
      mfma3(srow, __builtin_bit_cast(bf16x8_t, cur.dout[tb]), s0, s1);
      float gd[8], num[8], dr[8];
      unpack8(cur.dout[tb], gd);
      num[0] = n0[0], num[1] = n0[1], num[2] = n0[2], num[3] = n0[3];
      num[4] = n1[0], num[5] = n1[1], num[6] = n1[2], num[7] = n1[3];
      dr[0] = s0[0], dr[1] = s0[1], dr[2] = s0[2], dr[3] = s0[3];
      dr[4] = s1[0], dr[5] = s1[1], dr[6] = s1[2], dr[7] = s1[3];
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) dot += gd[j] * num[j];
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      const float dden = -dot * rden * rden;
#pragma unroll
      for (int j = 0; j < 8; ++j) dr[j] *= rden;
      if constexpr (ROPE) rotate8<true>(dr, ang_c, ang_s);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        dr[j] = pq[j] > 0.f ? dr[j] + zf[j] * dden : 0.f;
        dzacc[j] += pq[j] * dden;
      }
      store16_nt(rdq, out_off + tb * 16 * (int)orow, pack8(dr));
      // dnum (and phi~(Q)) of token row 16tb + n, features 8g .. 8g+7
      float* rowp = dn_tile + (16 * tb + n) * kTileRow + 8 * g;
      *reinterpret_cast<f32x4_t*>(rowp) = f32x4_t{gd[0] * rden, gd[1] * rden, gd[2] * rden, gd[3] * rden};
      *reinterpret_cast<f32x4_t*>(rowp + 4) = f32x4_t{gd[4] * rden, gd[5] * rden, gd[6] * rden, gd[7] * rden};
      if constexpr (ROPE) {
        float* rowq = pq_tile + (16 * tb + n) * kTileRow + 8 * g;
        *reinterpret_cast<f32x4_t*>(rowq) = f32x4_t{y[0], y[1], y[2], y[3]};
        *reinterpret_cast<f32x4_t*>(rowq + 4) = f32x4_t{y[4], y[5], y[6], y[7]};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // turned-around operands: lane (n, g), k-slots (tb, i) = tokens 16tb + 4g + i
    bf16x8_t bd[2][3];  // dnum, B operand for value half fh' (columns n)
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
      unsigned part[3][4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const float* col = dn_tile + (16 * tb + 4 * g) * kTileRow + 16 * fh + n;
        split3_bf16x2(col[0], col[kTileRow], part[0][2 * tb], part[1][2 * tb], part[2][2 * tb]);
        split3_bf16x2(col[2 * kTileRow], col[3 * kTileRow], part[0][2 * tb + 1], part[1][2 * tb + 1],
                      part[2][2 * tb + 1]);
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) bd[fh][k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
    }
    if constexpr (!ROPE) {
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        const bf16x8_t aq = pack_turned(turn(bq[0], sel[fh]), turn(bq[1], sel[fh]));
#pragma unroll
        for (int fv = 0; fv < 2; ++fv) {
          acc[fh][fv] = mfma16(aq, bd[fv][0], acc[fh][fv]);
          acc[fh][fv] = mfma16(aq, bd[fv][1], acc[fh][fv]);
          acc[fh][fv] = mfma16(aq, bd[fv][2], acc[fh][fv]);
        }
      }
    } else {
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        unsigned part[3][4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const float* col = pq_tile + (16 * tb + 4 * g) * kTileRow + 16 * fh + n;
          split3_bf16x2(col[0], col[kTileRow], part[0][2 * tb], part[1][2 * tb], part[2][2 * tb]);
          split3_bf16x2(col[2 * kTileRow], col[3 * kTileRow], part[0][2 * tb + 1], part[1][2 * tb + 1],
                        part[2][2 * tb + 1]);
        }
        bf16x8_t aq[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) aq[k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
#pragma unroll
        for (int fv = 0; fv < 2; ++fv) {
          f32x4_t x = acc[fh][fv];
          x = mfma16(aq[0], bd[fv][0], x);
          x = mfma16(aq[0], bd[fv][1], x);
          x = mfma16(aq[1], bd[fv][0], x);
          x = mfma16(aq[0], bd[fv][2], x);
          x = mfma16(aq[2], bd[fv][0], x);
          x = mfma16(aq[1], bd[fv][1], x);
          acc[fh][fv] = x;
        }
      }
    }
  }

  // dz: sum the 16 lanes of each group (token rows), feature 8g + j
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float x = dzacc[j];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    dzacc[j] = x;
  }
  // D lane (n, g): rows 4g + i -> key feature 16fh + 4g + i, column n -> value feature 16fh' + n
  float* rw = red[w];
#pragma unroll
  for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * fh + 4 * g + i;
      rw[d * 32 + n] = acc[fh][0][i];
      rw[d * 32 + 16 + n] = acc[fh][1][i];
    }
  }
  if (n == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) rw[1024 + 8 * g + j] = dzacc[j];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kStateElems; idx += kThreads)
    red[0][idx] = (red[0][idx] + red[1][idx]) + (red[2][idx] + red[3][idx]);
  __syncthreads();
  write_partial(red[0], bh, c, s, a);
}

}  // namespace la
