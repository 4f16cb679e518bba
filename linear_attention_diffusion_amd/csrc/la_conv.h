// Temporal convolution of the block-inference cache (gfx950).
//
// The Spatial-Temporal Mix-FFN alternates 1x3x3 spatial and 3x1x1 temporal
// filters ("SANA-Video" news article, "Design details"); the temporal conv
// enters through a shortcut ("SANA-Video" paper notes, section 3 Stage 2), and
// block inference keeps its last frame as the third part of the cache (paper
// notes, section 4).  Per channel c of every spatial token s:
//   y[b][f][s][c] = x[b][f][s][c] + w[c][0] x[b][f-1][s][c] + w[c][1] x[b][f][s][c]
//                   + w[c][2] x[b][f+1][s][c] + bias[c]
// with x[b][-1] = the cached last frame of the previous chunk (zeros without a
// cache) and x[b][F] = 0 (no later chunk exists yet).
//
// Layout x, y: [B][F][S][C] with C contiguous; cache: [B][S][C].  One thread
// per (b, s, 8 channels) column walks the F frames in blocks of four, every
// element read and written once; consecutive threads take consecutive
// 8-channel groups (one 16-byte bf16 piece each, coalesced).
#pragma once

#include "la_kernels.h"

namespace la {

// 8 channels of one frame as fp32
struct Vec8 {
  float v[8];
};

__device__ __forceinline__ Vec8 load8(const float* p) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
  return Vec8{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
}

__device__ __forceinline__ Vec8 load8(const __bf16* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  Vec8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.v[2 * j] = bf16lo_to_f32(x[j]);
    r.v[2 * j + 1] = bf16hi_to_f32(x[j]);
  }
  return r;
}

// The bf16 kernel keeps its loaded frames as raw 16-byte pieces and widens
// them to fp32 where they are used: a frame then holds 4 registers, not 8.
__device__ __forceinline__ u32x4_t load_raw(const __bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ Vec8 widen(u32x4_t x) {
  Vec8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.v[2 * j] = bf16lo_to_f32(x[j]);
    r.v[2 * j + 1] = bf16hi_to_f32(x[j]);
  }
  return r;
}

__device__ __forceinline__ void store8(float* p, const Vec8& x) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{x.v[0], x.v[1], x.v[2], x.v[3]};
  *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{x.v[4], x.v[5], x.v[6], x.v[7]};
}

__device__ __forceinline__ void store8(__bf16* p, const Vec8& x) {
  const u32x4_t o = {pack_bf16x2(x.v[0], x.v[1]), pack_bf16x2(x.v[2], x.v[3]), pack_bf16x2(x.v[4], x.v[5]),
                     pack_bf16x2(x.v[6], x.v[7])};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(p));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void temporal_conv3(const T* __restrict__ x, T* __restrict__ y,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias, const T* cache_in,
                                                           T* cache_out, int F, int64_t S, int C, int64_t cols) {
  const int64_t col = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (col >= cols) return;
  const int groups = C / 8;
  const int64_t bs = col / groups;
  const int c0 = (int)(col % groups) * 8;
  const int64_t b = bs / S;
  const int64_t s = bs % S;
  const int64_t frame = S * C;  // elements between frames
  const T* xc = x + b * F * frame + s * C + c0;
  T* yc = y + b * F * frame + s * C + c0;

  // the 8 channels' taps are 24 consecutive floats of w (16-byte aligned, as
  // c0 is a multiple of 8): six 16-byte loads
  float taps[24], w0[8], w1[8], w2[8], bb[8];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const f32x4_t t = *reinterpret_cast<const f32x4_t*>(w + c0 * 3 + 4 * i);
    taps[4 * i] = t[0];
    taps[4 * i + 1] = t[1];
    taps[4 * i + 2] = t[2];
    taps[4 * i + 3] = t[3];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w0[j] = taps[3 * j];
    w1[j] = taps[3 * j + 1];
    w2[j] = taps[3 * j + 2];
  }
  const Vec8 bv = bias ? load8(bias + c0) : Vec8{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < 8; ++j) bb[j] = bv.v[j];
  const int64_t cache_at = bs * C + c0;
  // blocks of kFrames frames: the block and its right neighbour are requested
  // together, so each thread keeps kFrames + 1 loads in flight
  constexpr int kFrames = 4;
  if constexpr (sizeof(T) == 2) {
    const u32x4_t zr = {0u, 0u, 0u, 0u};
    u32x4_t prev = cache_in ? load_raw(cache_in + cache_at) : zr;
    for (int f0 = 0; f0 < F; f0 += kFrames) {
      u32x4_t win[kFrames + 1];
#pragma unroll
      for (int u = 0; u <= kFrames; ++u) win[u] = (f0 + u < F) ? load_raw(xc + (f0 + u) * frame) : zr;
#pragma unroll
      for (int u = 0; u < kFrames; ++u) {
        if (f0 + u >= F) break;
        const Vec8 l = widen(u == 0 ? prev : win[u - 1]), m = widen(win[u]), r = widen(win[u + 1]);
        Vec8 out;
#pragma unroll
        for (int j = 0; j < 8; ++j) out.v[j] = m.v[j] + w0[j] * l.v[j] + w1[j] * m.v[j] + w2[j] * r.v[j] + bb[j];
        store8(yc + (f0 + u) * frame, out);
      }
      const int last = (F - f0 < kFrames ? F - f0 : kFrames) - 1;
#pragma unroll
      for (int u = 0; u < kFrames; ++u)
        if (u == last) prev = win[u];
    }
    // the last frame's own bits are the next chunk's cache; this thread read
    // the old cache entry first, so cache_out may be cache_in
    if (cache_out) __builtin_nontemporal_store(prev, reinterpret_cast<u32x4_t*>(cache_out + cache_at));
    return;
  }
  const Vec8 zero = {{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
  Vec8 prev = cache_in ? load8(cache_in + cache_at) : zero;
  for (int f0 = 0; f0 < F; f0 += kFrames) {
    Vec8 win[kFrames + 1];
#pragma unroll
    for (int u = 0; u <= kFrames; ++u) win[u] = (f0 + u < F) ? load8(xc + (f0 + u) * frame) : zero;
#pragma unroll
    for (int u = 0; u < kFrames; ++u) {
      if (f0 + u >= F) break;
      const Vec8& left = u == 0 ? prev : win[u - 1];
      Vec8 out;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        out.v[j] = win[u].v[j] + w0[j] * left.v[j] + w1[j] * win[u].v[j] + w2[j] * win[u + 1].v[j] + bb[j];
      store8(yc + (f0 + u) * frame, out);
    }
    const int last = (F - f0 < kFrames ? F - f0 : kFrames) - 1;
#pragma unroll
    for (int u = 0; u < kFrames; ++u)
      if (u == last) prev = win[u];
  }
  // `prev` is the column's last frame, the next chunk's cache; this thread
  // read the old cache entry first, so cache_out may be cache_in
  if (cache_out) store8(cache_out + cache_at, prev);
}

}  // namespace la
