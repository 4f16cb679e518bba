// Key/value projection fused with the state pass (gfx950 / CDNA4).
//
// Ahead of the attention, a layer projects its input x [B][N][C] into keys and
// values, K = x W_k^T and V = x W_v^T (per head, 32 features each).  Unfused,
// the projection GEMM writes K and V to HBM in bf16 and the state pass reads
// them back.  Here one kernel computes a head pair's K and V tiles with MFMA
// and contracts them into the heads' states on the spot, so K and V never
// reach memory (the fusion of ReLU(K)^T V into the QKV projection that the
// "Sana" research note lists under "Infra", there in an INT8 engine; here in
// bf16).  The tiles are rounded to bf16, as a bf16 projection would store
// them, and then contracted as in the state pass.
//
// GEMM: workgroup = 4 waves, tile = 256 tokens x 128 output columns (key and
// value features of heads h, h + 1), channel steps of 32.  The A tile (256 x
// 32 of x) and the B tile (128 x 32, rows of W_k and W_v) are staged in LDS,
// double-buffered, rows padded to 40 bf16; wave w owns tokens 128 (w & 1) ..
// +127 and head h + (w >> 1): 8 x 4 MFMA blocks of 16 x 16, 32 MFMAs a step.
// (Measured on the 4096 px layer: a 4-head tile at one workgroup per CU, a
// 64-channel step, and loads issued two steps ahead were all slower.)
//
// Epilogue: the accumulator block of tokens 16i .. 16i + 15 holds, in lane
// (n, g), tokens 4g + (0..3) of feature n -- the turned-around layout the
// state pass builds with selection MFMAs -- so two row blocks pack straight
// into the bf16 operands of S = phi(K)^T V and z = sum phi(K).
//
// Blocks of the (token range, head pair) grid are dealt to the XCDs in
// contiguous runs, and inside a run walk 4 token ranges per head pair: the
// workgroups resident on one XCD then share each x slice among several head
// pairs and each weight slice among 4 token ranges in its L2.
#pragma once

#include "la_kernels.h"

namespace la {

constexpr int kProjTokens = 256;   // tokens per workgroup block
constexpr int kProjGroupM = 4;     // token ranges walked together per head pair (measured best of 1..35)
constexpr int kProjChannelQuantum = 32;  // C must be a multiple of this
constexpr int kXcds = 8;

struct ProjArgs {
  const char* x;    // [B][N][C] bf16
  const char* wk;   // [H * 32][C] bf16: row h * 32 + d = key feature d of head h
  const char* wv;   // [H * 32][C] bf16: value features, same order
  int64_t N;        // tokens per batch
  int C;            // input channels (a multiple of 32)
  int H;
  int Hp;           // head pairs, ceil(H / 2)
  int64_t R;        // token ranges per batch
  int64_t T;        // blocks of kProjTokens per range
  int64_t M;        // B * R
};

// Block (range mi, pair pi) of the grid for workgroup `blk` of `G`.
__device__ __forceinline__ void proj_block(uint32_t blk, uint32_t G, int64_t M, int P, int64_t* mi, int* pi) {
  const uint32_t q = G / kXcds, rem = G % kXcds, xcd = blk % kXcds, slot = blk / kXcds;
  const uint32_t L = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
  const int64_t per_group = (int64_t)kProjGroupM * P;
  const int64_t first = (int64_t)(L / per_group) * kProjGroupM;
  const int64_t gsize = M - first < kProjGroupM ? M - first : kProjGroupM;
  const int64_t in = (int64_t)L % per_group;
  *mi = first + in % gsize;
  *pi = (int)(in / gsize);
}

// One workgroup per (token range, head pair): 4 waves, wave w takes tokens
// 128 (w & 1) .. +127 of each 256-token block and head h + (w >> 1) (64 output
// columns: 8 x 4 MFMA blocks of 16 x 16).  Two workgroups fit a CU (VGPRs,
// LDS), which the loads' latency needs.  Staging: thread tid moves 16-byte
// piece tid % 4 of A rows tid / 4 + 64 j and of B rows tid / 4 + 64 j; B row R
// is row R % 32 of head h + R / 64's key (bit 5 of R clear) or value weights.
__global__ __launch_bounds__(kThreads, 2) void project_state_bf16(ProjArgs p, StateArgs a) {
  constexpr int kRow = 40;                    // staged bf16 per row (32 + 8 pad: no bank conflicts)
  constexpr int kA = kProjTokens * kRow;      // bf16 per A buffer
  constexpr int kB = 128 * kRow;              // bf16 per B buffer
  __shared__ __attribute__((aligned(16))) __bf16 sa[2][kA];
  __shared__ __attribute__((aligned(16))) __bf16 sb[2][kB];

  int64_t mi;
  int pi;
  proj_block(blockIdx.x, gridDim.x, p.M, p.Hp, &mi, &pi);
  const int64_t b = mi / p.R;
  const int r = (int)(mi % p.R);
  const int h = 2 * pi;
  const int64_t bh = b * p.H + h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int th = w & 1, hh = w >> 1;
  const int row = p.C * 2;  // bytes per token row and per weight row

  const int piece = tid & 3;
  const int trow = tid >> 2;
  const int a_off = trow * row + piece * 16;
  const int b_off = (trow & 31) * row + piece * 16;
  const int heads_here = p.H - h < 2 ? p.H - h : 2;
  // waves 0, 1 stage key rows, waves 2, 3 value rows
  const rsrc_t rw = make_rsrc((w >> 1 ? p.wv : p.wk) + (int64_t)h * 32 * row, (int64_t)heads_here * 32 * row);
  const char* xb = p.x + b * p.N * (int64_t)row;

  const unsigned one2 = 0x3f803f80u;
  const bf16x8_t ones = as_bf16x8(one2, one2, one2, one2);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t S[2][2] = {{zero4, zero4}, {zero4, zero4}}, Z[2] = {zero4, zero4};

  const int nk = p.C / 32;
  const int64_t nblk = (p.N + kProjTokens - 1) / kProjTokens;
  const int64_t blk_end = ((int64_t)r + 1) * p.T < nblk ? ((int64_t)r + 1) * p.T : nblk;
  for (int64_t blk = (int64_t)r * p.T; blk < blk_end; ++blk) {
    const int64_t tok0 = blk * kProjTokens;
    // rows at or past N read as zero: their keys and values are 0 and add nothing
    const rsrc_t rx = make_rsrc(xb + tok0 * row, (p.N - tok0) * row);
    u32x4_t ga[4], gb[2];
    auto fetch = [&](int k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ga[j] = __builtin_bit_cast(u32x4_t, load16(rx, a_off + j * 64 * row + k * 64));
#pragma unroll
      for (int j = 0; j < 2; ++j) gb[j] = __builtin_bit_cast(u32x4_t, load16(rw, b_off + j * 32 * row + k * 64));
    };
    auto put = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x4_t*>(&sa[buf][(trow + 64 * j) * kRow + piece * 8]) = ga[j];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        *reinterpret_cast<u32x4_t*>(&sb[buf][(trow + 64 * j) * kRow + piece * 8]) = gb[j];
    };
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = zero4;

    // the previous block's last step ended with a barrier, so buffer 0 is free
    fetch(0);
    put(0);
    __syncthreads();
    for (int k = 0; k < nk; ++k) {
      const int buf = k & 1;
      if (k + 1 < nk) fetch(k + 1);
      bf16x8_t bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t*>(&sb[buf][(64 * hh + 16 * j + n) * kRow + 8 * g]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_t af =
            *reinterpret_cast<const bf16x8_t*>(&sa[buf][(128 * th + 16 * i + n) * kRow + 8 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af, bf[j], acc[i][j]);
      }
      if (k + 1 < nk) put(buf ^ 1);
      __syncthreads();
    }

    // acc[i][j], lane (n, g): tokens 128 th + 16 i + 4 g + (0..3) of the
    // block, column 16 j + n of head h + hh (j = 0, 1: key features; 2, 3:
    // value features).  Row blocks 2t, 2t + 1 make one 32-token contraction.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8_t ka[2], vb[2];
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        ka[fh] = __builtin_bit_cast(
            bf16x8_t, relu_bf16x8(__builtin_bit_cast(u32x4_t, pack_turned(acc[2 * t][fh], acc[2 * t + 1][fh]))));
        vb[fh] = pack_turned(acc[2 * t][2 + fh], acc[2 * t + 1][2 + fh]);
      }
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        Z[fh] = mfma16(ka[fh], ones, Z[fh]);
        S[fh][0] = mfma16(ka[fh], vb[0], S[fh][0]);
        S[fh][1] = mfma16(ka[fh], vb[1], S[fh][1]);
      }
    }
  }

  // the waves' sums to LDS (over the A buffers: every read of them ended at
  // the last step's barrier) as red[2 th + hh], the two token halves of each
  // head added, and each head's sum written as partial r
  float(*red)[kStateElems] = reinterpret_cast<float(*)[kStateElems]>(&sa[0][0]);
  float* mine = red[2 * th + hh];
#pragma unroll
  for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * fh + 4 * g + i;
      mine[d * 32 + n] = S[fh][0][i];
      mine[d * 32 + 16 + n] = S[fh][1][i];
      if (n == 0) mine[1024 + d] = Z[fh][i];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * kStateElems; idx += kThreads) red[0][idx] += red[2][idx];
  __syncthreads();
  write_partial(red[0], bh, 0, r, a);
  if (heads_here == 2) write_partial(red[1], bh + 1, 0, r, a);
}

}  // namespace la
