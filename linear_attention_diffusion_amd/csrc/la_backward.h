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
// These kernels keep the arithmetic in fp32 on the VALU, with Q/K/V/dO/dQ/dK/dV
// as fp32 or bf16 (converted on load, RNE on store).
#pragma once

#include "la_kernels.h"

namespace la {

// ---------------------------------------------------------------------------
// Element I/O: four consecutive features as fp32
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4_t load4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }

__device__ __forceinline__ f32x4_t load4(const __bf16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4_t{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
}

__device__ __forceinline__ void store4(float* p, f32x4_t x) { *reinterpret_cast<f32x4_t*>(p) = x; }

__device__ __forceinline__ void store4(__bf16* p, f32x4_t x) {
  *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}

// Sum over the 8 consecutive lanes that share a token
__device__ __forceinline__ float sum8(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

// Features f0 .. f0+3 (two pairs) of a token rotated by +theta (forward) or
// -theta (the transpose, on the way back).
template <bool INVERSE>
__device__ __forceinline__ f32x4_t rotate4(f32x4_t x, const float* cos_row, const float* sin_row, int f0) {
  f32x4_t y;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float c = cos_row[f0 / 2 + u];
    const float s = INVERSE ? -sin_row[f0 / 2 + u] : sin_row[f0 / 2 + u];
    y[2 * u] = x[2 * u] * c - x[2 * u + 1] * s;
    y[2 * u + 1] = x[2 * u] * s + x[2 * u + 1] * c;
  }
  return y;
}

// ---------------------------------------------------------------------------
// Reverse finalize: suffix sums of the query pass's partial state gradients
// ---------------------------------------------------------------------------
//
// One thread per state element of every head.  It starts from the gradient
// reaching the committed state (kv_in/ksum_in of `a`, or 0), walks the head's
// C x Pc partials from the last to the first, 16 loads in flight at a time,
// stores the running sum at the start of every chunk (G_c) and commits the
// total (G_0, the gradient of the carried state) to kv_out/ksum_out.
__global__ __launch_bounds__(kThreads) void state_finalize_reverse(StateArgs a, int64_t n_elems) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_elems) return;
  const int64_t bh = i / kStateElems;
  const int idx = (int)(i % kStateElems);
  const int total = a.C * a.Pc;
  const float* src = a.partials + bh * total * kStateElems + idx;
  float* dst = a.states + bh * a.C * kStateElems + idx;
  float acc = carried(a, bh, idx);
  for (int q0 = total - 1; q0 >= 0; q0 -= 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = (q0 - u >= 0) ? src[(int64_t)(q0 - u) * kStateElems] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int q = q0 - u;
      acc += v[u];
      if (q >= 0 && q % a.Pc == 0) dst[(int64_t)(q / a.Pc) * kStateElems] = acc;
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
template <typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void bwd_query_vec(const T* __restrict__ Q, const T* __restrict__ dO,
                                                          T* __restrict__ dQ, StateView fwd, float eps,
                                                          const float* __restrict__ cos_t,
                                                          const float* __restrict__ sin_t, int64_t pos0,
                                                          StateArgs a) {
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
  const int64_t N = a.N;
  const int t = threadIdx.x;
  const int tl = t >> 3;
  const int f0 = (t & 7) * 4;
  const int64_t sc = bh * a.C + c;
  for (int idx = t; idx < kD * kD; idx += kThreads) sS[idx >> 5][idx & 31] = fwd.s_base[sc * fwd.s_stride + idx];
  if (t < kD) sz[t] = fwd.z_base[sc * fwd.z_stride + t];

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  for (int64_t t0 = n_begin; t0 < n_end; t0 += 32) {
    const int64_t tok = t0 + tl;
    const bool live = tok < n_end;
    const int64_t row = (bh * N + tok) * kD + f0;
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
      if (live) pr = rotate4<false>(p, cos_t + (pos0 + tok) * 16, sin_t + (pos0 + tok) * 16, f0);
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
    const float rden = 1.f / den;
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
      if (live) dr = rotate4<true>(dr, cos_t + (pos0 + tok) * 16, sin_t + (pos0 + tok) * 16, f0);
    }
    f32x4_t dq;
#pragma unroll
    for (int u = 0; u < 4; ++u) dq[u] = x[u] > 0.f ? dr[u] + sz[f0 + u] * dden : 0.f;
    if (live) store4(dQ + row, dq);
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
template <typename T, bool ROPE>
__global__ __launch_bounds__(kThreads) void bwd_key_vec(const T* __restrict__ K, const T* __restrict__ V,
                                                        T* __restrict__ dK, T* __restrict__ dV, StateView grad,
                                                        int64_t N, int64_t L, int C, int tiles, int64_t Lt,
                                                        const float* __restrict__ cos_t,
                                                        const float* __restrict__ sin_t, int64_t pos0) {
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

  for (int64_t t0 = n_begin; t0 < n_end; t0 += 32) {
    const int64_t tok = t0 + tl;
    const bool live = tok < n_end;
    const int64_t row = (bh * N + tok) * kD + f0;
    f32x4_t x = {0.f, 0.f, 0.f, 0.f}, vv = x;
    if (live) {
      x = load4(K + row);
      vv = load4(V + row);
    }
    f32x4_t p;
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = fmaxf(x[u], 0.f);
    if constexpr (ROPE) {
      if (live) p = rotate4<false>(p, cos_t + (pos0 + tok) * 16, sin_t + (pos0 + tok) * 16, f0);
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
      if (live) dr = rotate4<true>(dr, cos_t + (pos0 + tok) * 16, sin_t + (pos0 + tok) * 16, f0);
    }
    f32x4_t dk;
#pragma unroll
    for (int u = 0; u < 4; ++u) dk[u] = x[u] > 0.f ? dr[u] + sGz[f0 + u] : 0.f;
    if (live) {
      store4(dK + row, dk);
      store4(dV + row, dv);
    }
  }
}

}  // namespace la
