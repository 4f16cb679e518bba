// Projections fused with the attention (gfx950 / CDNA4): keys and values with
// the state pass, queries with the apply pass.
//
// Ahead of the attention, a layer projects its input x [B][N][C] into keys and
// values, K = x W_k^T and V = x W_v^T (per head, 32 features each).  Unfused,
// the projection GEMM writes K and V to HBM in bf16 and the state pass reads
// them back.  Here one kernel computes four heads' K and V tiles with MFMA
// and contracts them into the heads' states on the spot, so K and V never
// reach memory (the fusion of ReLU(K)^T V into the QKV projection that the
// "Sana" research note lists under "Infra", there in an INT8 engine; here in
// bf16).  The tiles are rounded to bf16, as a bf16 projection would store
// them, and then contracted as in the state pass.
//
// GEMM: workgroup = 8 waves, tile = 256 tokens x 256 output columns (key and
// value features of heads h .. h + 3), channel steps of 32.  The A tile (256 x
// 32 of x) and the B tile (256 x 32, rows of W_k and W_v) go from memory
// straight into LDS (buffer loads with the lds flag: no staging registers, no
// LDS stores), in three stages, so step k + 2 loads while step k computes;
// wave w owns tokens 128 (w & 1) .. +127 and head h + (w >> 1): 8 x 4 MFMA
// blocks of 16 x 16, 32 MFMAs a step.  One workgroup fills a CU (96 KB of LDS;
// 2 waves per SIMD).  Measured against the earlier 4-wave, 256 x 128 tile at
// two workgroups per CU: the x tile now feeds four heads instead of two, and
// each step's LDS traffic per flop falls by an eighth.  (Also measured on the
// 4096 px layer: loads staged through registers into padded double-buffered
// LDS were 7% slower.)

// Epilogue: the accumulator block of tokens 16i .. 16i + 15 holds, in lane
// (n, g), tokens 4g + (0..3) of feature n -- the turned-around layout the
// state pass builds with selection MFMAs -- so two row blocks pack straight
// into the bf16 operands of S = phi(K)^T V and z = sum phi(K).  With RoPE,
// phi(K) is rotated in fp32 first (the pair partner comes from the
// neighbouring lane) and contracted as three bf16 parts; z stays unrotated.
//
// Blocks of the (token range, head group) grid are dealt to the XCDs in
// contiguous runs, and inside a run walk 4 token ranges per head group: the
// workgroups resident on one XCD then share each x slice among several head
// groups and each weight slice among 4 token ranges in its L2.
//
// The query side (project_apply_bf16, at the end) runs the same GEMM over eight
// heads' query weights and hands each 16-token tile of Q to the apply pass's
// arithmetic in registers.
#pragma once

#include "la_kernels.h"

namespace la {

constexpr int kProjTokens = 256;   // tokens per workgroup block
constexpr int kProjGroupM = 4;     // token ranges walked together per head group (measured best of 1..35)
constexpr int kProjChannelQuantum = 32;  // C must be a multiple of this
constexpr int kXcds = 8;
constexpr int kProjWaves = 8;                // waves per workgroup
constexpr int kProjThreads = 64 * kProjWaves;
constexpr int kProjCols = 32 * kProjWaves;   // B rows (output columns) per stage

struct ProjArgs {
  const char* x;    // [B][N][C] bf16
  const char* wk;   // [H * 32][C] bf16: row h * 32 + d = key feature d of head h
  const char* wv;   // [H * 32][C] bf16: value features, same order
  int64_t N;        // tokens per batch
  int C;            // input channels (a multiple of 32)
  int H;
  int Hp;           // head groups of four, ceil(H / 4)
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

// Loads x and weight rows straight into LDS (buffer_load ... lds): a wave's
// instruction fills 1 KB of LDS, 16 rows of 64 bytes (one 32-channel step),
// lane l writing row l / 4, slot l % 4.  Slots are XOR-swizzled: slot s of row
// r holds 16-byte piece s ^ swz(r) of the row, which makes the MFMA operand
// reads (16 rows, one piece each) free of bank conflicts with 32 or 64 banks.
__device__ __forceinline__ int proj_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ void lds_dma16(rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Waits until at most N of this wave's loads are outstanding (vmcnt(N)) and its
// LDS reads have completed (lgkmcnt(0)), then meets the other waves.  The
// acquire fence keeps later LDS reads below the barrier; no release fence, which
// would wait for every load in flight, the next stage's included.
template <int N>
__device__ __forceinline__ void proj_stage_barrier() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// cos/sin of this lane's two pairs (q[0], q[1]: features n and 16 + n) at
// position pos0 + tok (tok in the call's range): from the full tables in
// memory, or from the per-axis tables staged in LDS (rtab; ap: where each
// pair's entries sit), the coordinates computed once for both.
template <int ROPE>
__device__ __forceinline__ void proj_angles(const Rope& r, const float* rtab, const AxisPair (&ap)[2], int64_t tok,
                                            float (&c)[2], float (&sn)[2]) {
  const int64_t pos = r.pos0 + tok;
  if constexpr (ROPE == kRopeAxes) {
    int t, h, w;
    rope_coords(r, pos, t, h, w);
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
      axis_cs(rtab, axis_entry(ap[fh], t, h, w), c[fh], sn[fh]);
    }
  } else {
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
      const int q = (16 * fh + (int)(threadIdx.x & 15)) >> 1;
      c[fh] = r.cos[pos * 16 + q];
      sn[fh] = r.sin[pos * 16 + q];
    }
  }
}

// The GEMM of one 256-token block: acc[i][j] (lane (n, g): tokens
// 128 (w & 1) + 16 i + 4 g + (0..3), column 16 j + n of this wave's 64) over
// all nk 32-channel steps.  Three LDS stages of one step each (A: 256 token
// rows at 0, B: 256 weight rows at kProjBOff, 64 bytes a row); wave w's loads
// fill A rows 32 w .. 32 w + 31 (a_voff: row offsets in x, rsrc rx) and B rows
// 32 w .. 32 w + 31 (b_voff, rsrc rw); step k + 2 is loaded while step k
// computes.  Step t computes on stage t % 3.  Its barrier waits for the step's
// own loads (every wave's) to land and for step t - 1's reads to end
// everywhere; then stage (t + 2) % 3 is free for step t + 2's loads.  Each
// step issues four loads per wave, so with step t + 1's loads still in flight
// the wait is vmcnt(4), and vmcnt(0) at the last step.  In the main loop the
// stages are named, not indexed: the compiler then sees that the operand reads
// and the loads in flight touch different LDS arrays and adds no wait of its
// own, except at the loop head, where it cannot tell the stages apart across
// the back edge and waits for every load.  Six steps per iteration halve
// those waits (measured 3-4% faster than three; 24 steps were no faster).  The
// caller has synchronised the workgroup since the stages were last read.
constexpr int kProjStage = (kProjTokens + kProjCols) * 64;  // bytes per stage
constexpr int kProjBOff = kProjTokens * 64;            // B rows after the A rows

__device__ __forceinline__ void proj_gemm(rsrc_t rx, rsrc_t rw, const int (&a_voff)[2], const int (&b_voff)[2],
                                          int a_rd, int b_rd, int nk, int w, char* st0, char* st1, char* st2,
                                          f32x4_t (&acc)[8][4]) {
  auto issue = [&](int k, char* stage) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(rx, stage + (32 * w + 16 * i) * 64, a_voff[i] + k * 64);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(rw, stage + kProjBOff + (32 * w + 16 * i) * 64, b_voff[i] + k * 64);
  };
  auto compute = [&](const char* stage) {
    bf16x8_t bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const bf16x8_t*>(stage + b_rd + j * 1024);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(stage + a_rd + i * 1024);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af, bf[j], acc[i][j]);
    }
  };
  issue(0, st0);
  if (nk > 1) issue(1, st1);
  // steps k .. k + 2 (stages 0, 1, 2), every one with loads to issue
  auto three = [&](int k) {
    proj_stage_barrier<4>();
    issue(k + 2, st2);
    compute(st0);
    proj_stage_barrier<4>();
    issue(k + 3, st0);
    compute(st1);
    proj_stage_barrier<4>();
    issue(k + 4, st1);
    compute(st2);
  };
  int k = 0;
  for (; k + 8 <= nk; k += 6) {
    three(k);
    three(k + 3);
  }
  for (; k + 5 <= nk; k += 3) three(k);
  // the last 1 to 4 steps (k is a multiple of 3: step t is on stage t % 3)
  for (; k < nk; ++k) {
    const int sk = k % 3;
    char* cur = sk == 0 ? st0 : (sk == 1 ? st1 : st2);
    char* nxt = sk == 0 ? st2 : (sk == 1 ? st0 : st1);
    if (k + 1 < nk)
      proj_stage_barrier<4>();
    else
      proj_stage_barrier<0>();
    if (k + 2 < nk) issue(k + 2, nxt);
    compute(cur);
  }
}

// One workgroup per (token range, head group): 8 waves, wave w takes tokens
// 128 (w & 1) .. +127 of each 256-token block and head h + (w >> 1) (64 output
// columns: 8 x 4 MFMA blocks of 16 x 16) through proj_gemm.  B row R of a
// stage is row R % 32 of head h + R / 64's key (bit 5 of R clear) or value
// weights.  One workgroup fills a CU (96 KB of LDS, 104 KB with the per-axis
// RoPE tables).
template <int ROPE>
__global__ __launch_bounds__(kProjThreads, 1) void project_state_bf16(ProjArgs p, Rope rp, StateArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st1[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st2[kProjStage];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];

  int64_t mi;
  int pi;
  proj_block(blockIdx.x, gridDim.x, p.M, p.Hp, &mi, &pi);
  const int64_t b = mi / p.R;
  const int r = (int)(mi % p.R);
  const int h = 4 * pi;
  const int64_t bh = b * p.H + h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int th = w & 1, hh = w >> 1;
  const int row = p.C * 2;  // bytes per token row and per weight row

  // loads: lane l fills row l / 4 (of 16), slot l % 4, with the swizzled piece
  const int dr = lane >> 2;
  const int dpiece = ((lane & 3) ^ proj_swz(dr)) * 16;
  int a_voff[2], b_voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_voff[i] = (32 * w + 16 * i + dr) * row + dpiece;
  // wave w stages rows 32 w .. 32 w + 31 of B: features of head h + (w >> 1),
  // keys for even w, values for odd w
#pragma unroll
  for (int i = 0; i < 2; ++i) b_voff[i] = ((w >> 1) * 32 + 16 * i + dr) * row + dpiece;
  const int heads_here = p.H - h < 4 ? p.H - h : 4;
  const rsrc_t rw = make_rsrc((w & 1 ? p.wv : p.wk) + (int64_t)h * 32 * row, (int64_t)heads_here * 32 * row);
  const char* xb = p.x + b * p.N * (int64_t)row;
  // operand reads: lane (n, g) reads piece g of row base + n
  const int sw = 16 * (g ^ proj_swz(n));
  const int a_rd = (128 * th + n) * 64 + sw;
  const int b_rd = kProjBOff + (64 * hh + n) * 64 + sw;
  // RoPE: the pair partner's sign, and where the per-axis entries of this
  // lane's pairs (features n and 16 + n) sit; the axis tables go to LDS (the
  // first block's barrier orders the copy before any lookup)
  const float sgn = (n & 1) ? 1.f : -1.f;
  const AxisPair ap[2] = {axis_pair(rp, n >> 1), axis_pair(rp, (16 + n) >> 1)};
  rope_stage<ROPE>(rp, rtab, tid, kProjThreads);

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
    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = zero4;
    __syncthreads();  // every wave is done with the previous block's stages
    proj_gemm(rx, rw, a_voff, b_voff, a_rd, b_rd, nk, w, st0, st1, st2, acc);

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
      for (int fh = 0; fh < 2; ++fh) Z[fh] = mfma16(ka[fh], ones, Z[fh]);
      if constexpr (ROPE == kRopeNone) {
#pragma unroll
        for (int fh = 0; fh < 2; ++fh) {
          S[fh][0] = mfma16(ka[fh], vb[0], S[fh][0]);
          S[fh][1] = mfma16(ka[fh], vb[1], S[fh][1]);
        }
      } else {
        // Slot s of ka[fh] holds phi(K) of feature f = 16 fh + n for token
        // tok0 + 128 th + 16 (2t + s / 4) + 4 g + s % 4; the pair partner
        // f ^ 1 sits in lane n ^ 1, same slot.  Rotated: x c - x' s for even
        // f, x' s + x c for odd f, in fp32, then split into three bf16 parts
        // contracted against V one by one.  A token's angles are looked up
        // once for both feature halves.
        u32x4_t kw[2], pw[2];
#pragma unroll
        for (int fh = 0; fh < 2; ++fh) {
          kw[fh] = __builtin_bit_cast(u32x4_t, ka[fh]);
#pragma unroll
          for (int d = 0; d < 4; ++d) pw[fh][d] = (unsigned)__builtin_amdgcn_mov_dpp((int)kw[fh][d], 0xB1, 0xF, 0xF, false);
        }
        unsigned part[2][3][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float y[2][2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int slot = 2 * d + e;
            const int64_t tok = tok0 + 128 * th + 16 * (2 * t + (slot >> 2)) + 4 * g + (slot & 3);
            float c[2], sn[2];
            proj_angles<ROPE>(rp, rtab, ap, tok < p.N ? tok : p.N - 1, c, sn);
#pragma unroll
            for (int fh = 0; fh < 2; ++fh) {
              const float x = e ? bf16hi_to_f32(kw[fh][d]) : bf16lo_to_f32(kw[fh][d]);
              const float xp = sgn * (e ? bf16hi_to_f32(pw[fh][d]) : bf16lo_to_f32(pw[fh][d]));
              y[fh][e] = __builtin_fmaf(x, c[fh], xp * sn[fh]);  // the fusion fixed, as in rot_lo
            }
          }
#pragma unroll
          for (int fh = 0; fh < 2; ++fh) split3_bf16x2(y[fh][0], y[fh][1], part[fh][0][d], part[fh][1][d], part[fh][2][d]);
        }
#pragma unroll
        for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const bf16x8_t ar = as_bf16x8(part[fh][k][0], part[fh][k][1], part[fh][k][2], part[fh][k][3]);
            S[fh][0] = mfma16(ar, vb[0], S[fh][0]);
            S[fh][1] = mfma16(ar, vb[1], S[fh][1]);
          }
        }
      }
    }
  }

  // the waves' sums to LDS (over stages 0 and 1: no load is in flight after
  // the last step), token half th of head hh as red_th[hh]; the halves are
  // added and each head's sum is written as partial r
  __syncthreads();
  float(*red0)[kStateElems] = reinterpret_cast<float(*)[kStateElems]>(st0);
  float(*red1)[kStateElems] = reinterpret_cast<float(*)[kStateElems]>(st1);
  float* mine = (th ? red1 : red0)[hh];
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
  for (int idx = tid; idx < 4 * kStateElems; idx += kProjThreads) red0[0][idx] += red1[0][idx];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hq = 2 * j + (tid >> 8);
    if (hq < heads_here) write_partial(red0[hq], bh + hq, 0, r, a, tid & 255);
  }
}

// ---------------------------------------------------------------------------
// Query projection fused with the apply pass
// ---------------------------------------------------------------------------
//
// Q = x W_q^T through the same GEMM (eight heads of 32 query features per
// workgroup: wave w takes tokens 128 (w & 1) .. +127 and heads h + 2 (w >> 1)
// and h + 2 (w >> 1) + 1), rounded to bf16 as a bf16 projection would store
// it, and applied to the heads' states in the epilogue, so Q never reaches
// memory: O = phi~(Q).S / (phi(Q).z + eps).  The apply pass takes phi(Q) as an
// MFMA B operand with a token in each column; the GEMM leaves it turned
// around (a feature in each lane), so a selection MFMA turns each pair of
// 16-token blocks back, exactly (bf16 values times 1.0), with a lane's k-slots
// s holding features 4g + s (s < 4) and 16 + 4g + s - 4 (s >= 4); the S and z
// operands are loaded in that order, and apply_tile does the rest.

struct ProjApplyArgs {
  const char* x;     // [B][N][C] bf16
  const char* wq;    // [H * 32][C] bf16: row h * 32 + d = query feature d of head h
  char* o;           // outputs, bf16, through lo
  Layout lo;
  const float* kv;   // states [B * H][32][32] fp32
  const float* ks;   // [B * H][32] fp32
  int64_t N;
  int C;
  int H;
  int Hq;            // head groups of eight, ceil(H / 8)
  int64_t R;         // 256-token blocks per batch
  int64_t M;         // B * R
  float eps;
};

// B operand that picks, from a turned-around pair of 16-token blocks (k-slot
// s of lane g: token 4g + s % 4 of block s / 4), block bb's tokens in natural
// order: slot s of lane (n, g) is 1.0 where s / 4 == bb and 4g + s % 4 == n.
__device__ __forceinline__ bf16x8_t untangle_select(int g, int n, int bb) {
  unsigned d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s0 = 2 * q, s1 = 2 * q + 1;
    const bool h0 = (s0 >> 2) == bb && 4 * g + (s0 & 3) == n;
    const bool h1 = (s1 >> 2) == bb && 4 * g + (s1 & 3) == n;
    d[q] = (h0 ? 0x3f80u : 0u) | (h1 ? 0x3f800000u : 0u);
  }
  return as_bf16x8(d[0], d[1], d[2], d[3]);
}

// apply_tile's S^T and z operands (see load_apply_operands) for B operands
// whose k-slot s holds feature 4g + s (s < 4) or 16 + 4g + s - 4 (s >= 4).
__device__ __forceinline__ void proj_apply_operands(const float* S, const float* z, int g, int m,
                                                    ApplyOperands& op) {
  auto feat = [&](int s) { return s < 4 ? 4 * g + s : 12 + 4 * g + s; };
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int e = 8 * (m >> 2) + 4 * hf + (m & 3);
    unsigned part[3][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      split3_bf16x2(S[feat(2 * q) * 32 + e], S[feat(2 * q + 1) * 32 + e], part[0][q], part[1][q], part[2][q]);
#pragma unroll
    for (int k = 0; k < 3; ++k) op.s[hf][k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
  }
  unsigned part[3][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    split3_bf16x2(z[feat(2 * q)], z[feat(2 * q + 1)], part[0][q], part[1][q], part[2][q]);
#pragma unroll
  for (int k = 0; k < 3; ++k) op.z[k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
}

// One workgroup per (256-token block, group of eight heads).
template <int ROPE>
__global__ __launch_bounds__(kProjThreads, 1) void project_apply_bf16(ProjApplyArgs p, Rope rp) {
  __shared__ __attribute__((aligned(1024))) char st0[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st1[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st2[kProjStage];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];

  int64_t mi;
  int pi;
  proj_block(blockIdx.x, gridDim.x, p.M, p.Hq, &mi, &pi);
  const int64_t b = mi / p.R;
  const int64_t tok0 = (mi % p.R) * kProjTokens;
  const int h = 8 * pi;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int th = w & 1, hh = w >> 1;
  const int row = p.C * 2;

  const int dr = lane >> 2;
  const int dpiece = ((lane & 3) ^ proj_swz(dr)) * 16;
  int a_voff[2], b_voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_voff[i] = (32 * w + 16 * i + dr) * row + dpiece;
  // wave w stages B rows 32 w .. 32 w + 31: the query weights of head h + w
#pragma unroll
  for (int i = 0; i < 2; ++i) b_voff[i] = (32 * w + 16 * i + dr) * row + dpiece;
  const int heads_here = p.H - h < 8 ? p.H - h : 8;
  const rsrc_t rw = make_rsrc(p.wq + (int64_t)h * 32 * row, (int64_t)heads_here * 32 * row);
  // rows at or past N read as zero; their outputs are not stored
  const rsrc_t rx = make_rsrc(p.x + (b * p.N + tok0) * (int64_t)row, (p.N - tok0) * row);
  const int sw = 16 * (g ^ proj_swz(n));
  const int a_rd = (128 * th + n) * 64 + sw;
  const int b_rd = kProjBOff + (64 * hh + n) * 64 + sw;
  // RoPE: this lane's pairs are 2g, 2g + 1, 8 + 2g, 9 + 2g (its k-slot pairs),
  // two duos of the staged tables (pair counts per axis are even)
  const AxisPair ap[2] = {axis_pair(rp, 2 * g), axis_pair(rp, 8 + 2 * g)};
  rope_stage<ROPE>(rp, rtab, tid, kProjThreads);

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4;
  __syncthreads();  // the RoPE tables are staged
  proj_gemm(rx, rw, a_voff, b_voff, a_rd, b_rd, p.C / 32, w, st0, st1, st2, acc);

  // acc[i][2u + fh], lane (n, g): tokens 128 th + 16 i + 4 g + (0..3),
  // feature 16 fh + n of head h + 2 hh + u
  const bf16x8_t sel[2] = {untangle_select(g, n, 0), untangle_select(g, n, 1)};
  const int64_t tw0 = tok0 + 128 * th;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int hu = h + 2 * hh + u;
    if (hu >= p.H) break;
    const int64_t bh = b * p.H + hu;
    ApplyOperands op;
    proj_apply_operands(p.kv + bh * 1024, p.ks + bh * 32, g, n, op);
    const int64_t orow = p.lo.token * 2;
    const rsrc_t ro = rows_rsrc(p.o + p.lo.base(bh) * 2, tw0, p.N, orow);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8_t A[2];
#pragma unroll
      for (int fh = 0; fh < 2; ++fh)
        A[fh] = __builtin_bit_cast(bf16x8_t, relu_bf16x8(__builtin_bit_cast(
                                                 u32x4_t, pack_turned(acc[2 * t][2 * u + fh], acc[2 * t + 1][2 * u + fh]))));
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const f32x4_t d0 = mfma16(A[0], sel[bb], zero4), d1 = mfma16(A[1], sel[bb], zero4);
        const u32x4_t q = {pack_bf16x2(d0[0], d0[1]), pack_bf16x2(d0[2], d0[3]), pack_bf16x2(d1[0], d1[1]),
                           pack_bf16x2(d1[2], d1[3])};
        const int tr = 16 * (2 * t + bb) + n;  // this lane's token row in the wave's 128
        f32x4_t c = zero4, sn = zero4;
        if constexpr (ROPE != kRopeNone) {
          const int64_t tok = tw0 + tr < p.N ? tw0 + tr : p.N - 1;
          const int64_t pos = rp.pos0 + tok;
          if constexpr (ROPE == kRopeAxes) {
            int ct, chh, cw;
            rope_coords(rp, pos, ct, chh, cw);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const f32x4_t e = axis_duo(rtab, axis_entry(ap[d], ct, chh, cw));
              c[2 * d] = e[0];
              c[2 * d + 1] = e[1];
              sn[2 * d] = e[2];
              sn[2 * d + 1] = e[3];
            }
          } else {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int pq = (q4 < 2 ? 2 * g : 6 + 2 * g) + q4;
              c[q4] = rp.cos[pos * 16 + pq];
              sn[q4] = rp.sin[pos * 16 + pq];
            }
          }
        }
        store16_nt(ro, tr * (int)orow + 16 * g, apply_tile<ROPE != kRopeNone>(q, op, p.eps, c, sn));
      }
    }
  }
}

}  // namespace la
