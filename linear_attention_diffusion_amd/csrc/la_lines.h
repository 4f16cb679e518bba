// Two adjacent heads read as whole 128-byte lines (gfx950 / CDNA4).
//
// In a [B][N][H][D] view, or the q, k, v parts of a packed [B][N][3][H][D]
// projection output, heads 2u and 2u + 1 of a token are adjacent 64-byte
// rows: one 128-byte line.  The one-head kernels read such a layout in half
// lines, and on this part a half-line read costs a 64-byte request to HBM:
// the same bytes in twice the requests, and nearly twice the time.  These
// variants give a workgroup the head pair (2u, 2u + 1) (H even, so a pair never
// straddles two batches).  Each wave loads whole lines: lane l of a load takes
// the 16-byte piece l % 8 of token l / 8's line, so one load covers 8 tokens of
// both heads.  It then hands each head its natural tile through a wave-private
// LDS staging area (token rows of 36 floats: both heads' 32 features and 4 of
// padding against bank conflicts).
//
// Per head, the tiles, the order in which a wave takes them and the sums are
// those of the one-head kernels, so the results are bit-identical.
#pragma once

#include "la_backward.h"
#include "la_kernels.h"

namespace la {

constexpr int kLineRow = 36;              // staged floats per token
constexpr int kLineTile = 32 * kLineRow;  // one 32-token staging tile (4.5 KB)

// 32 tokens x 128 bytes from the descriptor's start: load j holds tokens 8j + l / 8.
__device__ __forceinline__ void load_lines(rsrc_t r, int line_off, int64_t row, u32x4_t (&x)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = load16_nt(r, line_off + j * 8 * (int)row);
}

// Descriptor for the lines of rows t0 .. n_end-1 (both heads, 128 bytes each).
__device__ __forceinline__ rsrc_t lines_rsrc(const char* pair_base, int64_t t0, int64_t n_end, int64_t row) {
  return make_rsrc(pair_base + t0 * row, (n_end - t0 - 1) * row + 128);
}

// The wave writes its 32 loaded lines to its staging tile and reads back the
// pieces it needs.  The wavefront-scope fences keep the compiler from moving
// LDS accesses across them (a wave's LDS accesses are performed in order).
__device__ __forceinline__ void stage_lines(float* st, int lane, const u32x4_t (&x)[4]) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<u32x4_t*>(st + (8 * j + (lane >> 3)) * kLineRow + (lane & 7) * 4) = x[j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Head hd's 16 bytes for lane (n, g) of 16-token half tb: features 8g .. 8g+7
// of token 16tb + n, as a one-head kernel would have loaded them.
__device__ __forceinline__ u32x4_t staged_piece(const float* st, int tb, int hd, int n, int g) {
  return *reinterpret_cast<const u32x4_t*>(st + (16 * tb + n) * kLineRow + hd * 16 + g * 4);
}

__device__ __forceinline__ void put_piece(float* st, int tb, int hd, int n, int g, u32x4_t x) {
  *reinterpret_cast<u32x4_t*>(st + (16 * tb + n) * kLineRow + hd * 16 + g * 4) = x;
}

// The staged tile back as whole lines (the inverse of stage_lines).
__device__ __forceinline__ void unstage_lines(const float* st, int lane, u32x4_t (&x)[4]) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x[j] = *reinterpret_cast<const u32x4_t*>(st + (8 * j + (lane >> 3)) * kLineRow + (lane & 7) * 4);
}

// ---------------------------------------------------------------------------
// State pass.  Workgroup (u, c, s) = blockIdx.x, numbered head-pair-minor
// (workgroups launched together read the same tokens), reduces tokens
// [s*Ls, ...) of chunk c for heads 2u and 2u + 1.  Wave w takes the 32-token
// tiles of the one-head kernel's wave w (64-token chunks at n_begin + 64w,
// step 256, first tile then second), for both heads.
// ---------------------------------------------------------------------------
template <int ROPE>
__global__ __launch_bounds__(kThreads) void state_bf16_lines(const u32x4_t* __restrict__ K,
                                                             const u32x4_t* __restrict__ V, Layout lkv, Rope rp,
                                                             StateArgs a, int64_t units) {
  // staging tiles (K, V per wave) during the loop, then the per-wave partial
  // states of both heads for the reduction
  constexpr int kStage = 4 * 2 * kLineTile;
  constexpr int kRed = 2 * 4 * kStateElems;
  __shared__ __attribute__((aligned(16))) float smem[kStage > kRed ? kStage : kRed];
  __shared__ float angles[ROPE ? 4 : 1][ROPE ? kAngTile : 1];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  int64_t u, n_begin, n_end;
  int c, s;
  state_item(a, u, c, s, n_begin, n_end, units);
  const int64_t bh0 = 2 * u;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only

  const int64_t row = lkv.token * 2;  // bytes between tokens
  const char* Kp = reinterpret_cast<const char*>(K) + lkv.base(bh0) * 2;
  const char* Vp = reinterpret_cast<const char*>(V) + lkv.base(bh0) * 2;
  const int line_off = (lane >> 3) * (int)row + (lane & 7) * 16;
  const int tab_off = n * 64 + g * 16;
  float* stk = smem + w * 2 * kLineTile;
  float* stv = stk + kLineTile;

  const bf16x8_t sel[2] = {select_operand(g, n, 0), select_operand(g, n, 1)};
  const bf16x8_t selp[2] = {partner_operand(g, n, 0), partner_operand(g, n, 1)};
  f32x4_t acc[2][2][2], accz[2][2];  // [head][...] as in the one-head kernel
#pragma unroll
  for (int hd = 0; hd < 2; ++hd)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      accz[hd][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc[hd][i][0] = accz[hd][i];
      acc[hd][i][1] = accz[hd][i];
    }

  u32x4_t nk[4], nv[4];
  TileAnglesRows na;  // cos/sin rows of the tile (full tables)
  auto load_tile = [&](int64_t t) {
    load_lines(lines_rsrc(Kp, t, n_end, row), line_off, row, nk);
    load_lines(lines_rsrc(Vp, t, n_end, row), line_off, row, nv);
    if constexpr (ROPE == kRopeTable) load_angle_rows(rp.cos, rp.sin, rp.pos0, t, n_end, tab_off, na);
  };
  float* lds = angles[ROPE ? w : 0];
  // the tiles of the wave: t0, t0 + 32, t0 + 256, t0 + 288, ... below n_end
  int64_t t = n_begin + 64 * w;
  if (t < n_end) load_tile(t);
  while (t < n_end) {
    const bool first = ((t - n_begin) & 63) == 0;
    const int64_t next = first ? t + 32 : t + 224;
    stage_lines(stk, lane, nk);
    stage_lines(stv, lane, nv);
    TileAnglesRows ra = na;
    if (next < n_end) load_tile(next);
    if constexpr (ROPE == kRopeAxes) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) rope_axis_row4(rp, rtab, al, rp.pos0 + t + 16 * tb + n, ra.c[tb], ra.s[tb]);
    }
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
      const u32x4_t kx[2] = {staged_piece(stk, 0, hd, n, g), staged_piece(stk, 1, hd, n, g)};
      const u32x4_t vx[2] = {staged_piece(stv, 0, hd, n, g), staged_piece(stv, 1, hd, n, g)};
      state_tile<ROPE != 0>(kx, vx, ra, g, n, lds, sel, selp, acc[hd], accz[hd]);
    }
    t = next;
  }

  __syncthreads();  // the reduction area overlaps other waves' staging tiles
  float(*red)[4][kStateElems] = reinterpret_cast<float(*)[4][kStateElems]>(smem);
#pragma unroll
  for (int hd = 0; hd < 2; ++hd) {
    float* rw = red[hd][w];
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * fh + 4 * g + i;
        rw[d * 32 + n] = acc[hd][fh][0][i];
        rw[d * 32 + 16 + n] = acc[hd][fh][1][i];
        if (n == 0) rw[1024 + d] = accz[hd][fh][i];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * kStateElems; idx += kThreads) {
    float(*r)[kStateElems] = red[idx / kStateElems];
    const int e = idx % kStateElems;
    r[0][e] = (r[0][e] + r[1][e]) + (r[2][e] + r[3][e]);
  }
  __syncthreads();
  write_partial(red[0][0], bh0, c, s, a);
  write_partial(red[1][0], bh0 + 1, c, s, a);
}

// ---------------------------------------------------------------------------
// Apply pass.  Workgroup blockIdx.x = blk * units + u takes tokens
// [blk * La, (blk + 1) * La) of heads 2u and 2u + 1, cut at chunk boundaries;
// wave w takes 32-token steps at n_begin + 32w, step 128, both heads, the
// state operands of both heads in registers.  When the output pairs heads too,
// each lane puts its outputs where it read its inputs in the staging tile, and
// the wave stores whole lines; otherwise it stores each head's rows.
// ---------------------------------------------------------------------------
template <int ROPE>
__global__ __launch_bounds__(kThreads) void apply_bf16_lines(const u32x4_t* __restrict__ Q, u32x4_t* __restrict__ O,
                                                             Layout lq, Layout lo, StateView sv, int64_t N,
                                                             int64_t L, int C, int64_t La, float eps, Rope rp,
                                                             int64_t units) {
  __shared__ __attribute__((aligned(16))) float smem[4 * kLineTile];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only
  const int64_t qrow = lq.token * 2, orow = lo.token * 2;  // bytes between tokens
  const int line_off = (lane >> 3) * (int)qrow + (lane & 7) * 16;
  const int o_off = m * (int)orow + g * 16;
  const int tab_off = m * 64 + g * 16;
  float* st = smem + w * kLineTile;

  const int64_t u = blockIdx.x % units;
  const int64_t f_begin = u * N + (int64_t)(blockIdx.x / units) * La;
  const int64_t f_end = (f_begin + La < (u + 1) * N) ? f_begin + La : (u + 1) * N;
  const int64_t bh0 = 2 * u;
  const char* Qp = reinterpret_cast<const char*>(Q) + lq.base(bh0) * 2;
  char* Oh[2] = {reinterpret_cast<char*>(O) + lo.base(bh0) * 2, reinterpret_cast<char*>(O) + lo.base(bh0 + 1) * 2};
  const bool out_lines = lo.head == kD;
  const int oline_off = (lane >> 3) * (int)orow + (lane & 7) * 16;

  // segments inside one chunk
  for (int64_t f = f_begin; f < f_end;) {
    const int64_t n_begin = f - u * N;
    const int c = (int)(n_begin / L);
    const int64_t c_end = ((int64_t)c + 1) * L < N ? ((int64_t)c + 1) * L : N;
    const int64_t n_end = (f_end - u * N < c_end) ? f_end - u * N : c_end;
    f = u * N + n_end;

    int64_t t0 = n_begin + 32 * w;
    u32x4_t nq[4];
    f32x4_t nc[2], ns[2];  // cos/sin rows of the step (full tables)
    auto load_step = [&](int64_t t) {
      load_lines(lines_rsrc(Qp, t, n_end, qrow), line_off, qrow, nq);
      if constexpr (ROPE == kRopeTable) {
        const rsrc_t rc = make_rsrc(rp.cos + (rp.pos0 + t) * 16, (n_end - t) * 64);
        const rsrc_t rs = make_rsrc(rp.sin + (rp.pos0 + t) * 16, (n_end - t) * 64);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          nc[tb] = load16(rc, tab_off + tb * 1024);
          ns[tb] = load16(rs, tab_off + tb * 1024);
        }
      }
    };
    if (t0 < n_end) load_step(t0);
    ApplyOperands op[2];
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
      const int64_t sc = (bh0 + hd) * C + c;
      load_apply_operands(sv.s_base + sc * sv.s_stride, sv.z_base + sc * sv.z_stride, g, m, op[hd]);
    }

    for (; t0 < n_end; t0 += 128) {
      stage_lines(st, lane, nq);
      f32x4_t cc[2] = {nc[0], nc[1]}, ss[2] = {ns[0], ns[1]};
      if (t0 + 128 < n_end) load_step(t0 + 128);
      if constexpr (ROPE == kRopeAxes) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 16 * tb + m, cc[tb], ss[tb]);
      }
      if (out_lines) {
#pragma unroll
        for (int hd = 0; hd < 2; ++hd)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            put_piece(st, tb, hd, m, g,
                      apply_tile<ROPE != 0>(staged_piece(st, tb, hd, m, g), op[hd], eps, cc[tb], ss[tb]));
        u32x4_t ol[4];
        unstage_lines(st, lane, ol);
        const rsrc_t ro = lines_rsrc(Oh[0], t0, n_end, orow);
#pragma unroll
        for (int j = 0; j < 4; ++j) store16_nt(ro, oline_off + j * 8 * (int)orow, ol[j]);
      } else {
#pragma unroll
        for (int hd = 0; hd < 2; ++hd) {
          const rsrc_t ro = rows_rsrc(Oh[hd], t0, n_end, orow);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            store16_nt(ro, o_off + tb * 16 * (int)orow,
                       apply_tile<ROPE != 0>(staged_piece(st, tb, hd, m, g), op[hd], eps, cc[tb], ss[tb]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key pass of the backward (dV = G^T phi~(K), dK = [K > 0] (R^T G V + Gz)),
// split like the apply pass: 32-token steps of both heads per wave, each
// head's G operands in registers.  Each lane puts its dK and dV pieces where it
// read the K and V pieces, so paired outputs leave as whole lines too.
// ---------------------------------------------------------------------------
template <int ROPE>
__global__ __launch_bounds__(kThreads) void bwd_key_bf16_lines(const u32x4_t* __restrict__ K,
                                                               const u32x4_t* __restrict__ V,
                                                               u32x4_t* __restrict__ dK, u32x4_t* __restrict__ dV,
                                                               Layout lin, Layout lout, StateView grad, int64_t N,
                                                               int64_t L, int C, int64_t La, Rope rp,
                                                               int64_t units) {
  __shared__ __attribute__((aligned(16))) float smem[4 * 2 * kLineTile];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only
  const int64_t irow = lin.token * 2, orow = lout.token * 2;  // bytes between tokens
  const int line_off = (lane >> 3) * (int)irow + (lane & 7) * 16;
  const int oline_off = (lane >> 3) * (int)orow + (lane & 7) * 16;
  const int o_off = m * (int)orow + g * 16;
  const int tab_off = m * 64 + g * 16;
  float* stk = smem + w * 2 * kLineTile;
  float* stv = stk + kLineTile;

  const int64_t u = blockIdx.x % units;
  const int64_t f_begin = u * N + (int64_t)(blockIdx.x / units) * La;
  const int64_t f_end = (f_begin + La < (u + 1) * N) ? f_begin + La : (u + 1) * N;
  const int64_t bh0 = 2 * u;
  const char* Kp = reinterpret_cast<const char*>(K) + lin.base(bh0) * 2;
  const char* Vp = reinterpret_cast<const char*>(V) + lin.base(bh0) * 2;
  char* dKh[2] = {reinterpret_cast<char*>(dK) + lout.base(bh0) * 2, reinterpret_cast<char*>(dK) + lout.base(bh0 + 1) * 2};
  char* dVh[2] = {reinterpret_cast<char*>(dV) + lout.base(bh0) * 2, reinterpret_cast<char*>(dV) + lout.base(bh0 + 1) * 2};
  const bool out_lines = lout.head == kD;

  for (int64_t f = f_begin; f < f_end;) {
    const int64_t n_begin = f - u * N;
    const int c = (int)(n_begin / L);
    const int64_t c_end = ((int64_t)c + 1) * L < N ? ((int64_t)c + 1) * L : N;
    const int64_t n_end = (f_end - u * N < c_end) ? f_end - u * N : c_end;
    f = u * N + n_end;

    int64_t t0 = n_begin + 32 * w;
    u32x4_t nk[4], nv[4];
    f32x4_t nc[2], ns[2];  // cos/sin rows of the step (full tables)
    auto load_step = [&](int64_t t) {
      load_lines(lines_rsrc(Kp, t, n_end, irow), line_off, irow, nk);
      load_lines(lines_rsrc(Vp, t, n_end, irow), line_off, irow, nv);
      if constexpr (ROPE == kRopeTable) {
        const rsrc_t rc = make_rsrc(rp.cos + (rp.pos0 + t) * 16, (n_end - t) * 64);
        const rsrc_t rs = make_rsrc(rp.sin + (rp.pos0 + t) * 16, (n_end - t) * 64);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          nc[tb] = load16(rc, tab_off + tb * 1024);
          ns[tb] = load16(rs, tab_off + tb * 1024);
        }
      }
    };
    if (t0 < n_end) load_step(t0);
    bf16x8_t gcol[2][2][3], grow[2][2][3];
    float gz[2][8];
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
      const int64_t sc = (bh0 + hd) * C + c;
      const float* G = grad.s_base + sc * grad.s_stride;
      const float* Gz = grad.z_base + sc * grad.z_stride;
      load_column_operands(G, g, m, gcol[hd]);  // dV = G^T phi~(K)
      load_row_operands(G, g, m, grow[hd]);     // G V
#pragma unroll
      for (int j = 0; j < 8; ++j) gz[hd][j] = Gz[8 * g + j];
    }

    for (; t0 < n_end; t0 += 128) {
      stage_lines(stk, lane, nk);
      stage_lines(stv, lane, nv);
      f32x4_t cc[2] = {nc[0], nc[1]}, ss[2] = {ns[0], ns[1]};
      if (t0 + 128 < n_end) load_step(t0 + 128);
      if constexpr (ROPE == kRopeAxes) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 16 * tb + m, cc[tb], ss[tb]);
      }
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        const rsrc_t rdk = rows_rsrc(dKh[hd], t0, n_end, orow);
        const rsrc_t rdv = rows_rsrc(dVh[hd], t0, n_end, orow);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const u32x4_t kr = relu_bf16x8(staged_piece(stk, tb, hd, m, g));
          const u32x4_t vx = staged_piece(stv, tb, hd, m, g);
          f32x4_t o0, o1;
          float x[8];
          if constexpr (ROPE == kRopeNone) {
            mfma3(gcol[hd], __builtin_bit_cast(bf16x8_t, kr), o0, o1);
          } else {
            float y[8];
            unpack8(kr, y);
            rotate8<false>(y, cc[tb], ss[tb]);
            bf16x8_t b[3];
            split8(y, b);
            mfma6(gcol[hd], b, o0, o1);
          }
          x[0] = o0[0], x[1] = o0[1], x[2] = o0[2], x[3] = o0[3];
          x[4] = o1[0], x[5] = o1[1], x[6] = o1[2], x[7] = o1[3];
          const u32x4_t dv_out = pack8(x);
          mfma3(grow[hd], __builtin_bit_cast(bf16x8_t, vx), o0, o1);
          x[0] = o0[0], x[1] = o0[1], x[2] = o0[2], x[3] = o0[3];
          x[4] = o1[0], x[5] = o1[1], x[6] = o1[2], x[7] = o1[3];
          if constexpr (ROPE != kRopeNone) rotate8<true>(x, cc[tb], ss[tb]);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            x[2 * p] = (kr[p] & 0xffffu) ? x[2 * p] + gz[hd][2 * p] : 0.f;
            x[2 * p + 1] = (kr[p] >> 16) ? x[2 * p + 1] + gz[hd][2 * p + 1] : 0.f;
          }
          const u32x4_t dk_out = pack8(x);
          if (out_lines) {
            put_piece(stk, tb, hd, m, g, dk_out);
            put_piece(stv, tb, hd, m, g, dv_out);
          } else {
            store16_nt(rdk, o_off + tb * 16 * (int)orow, dk_out);
            store16_nt(rdv, o_off + tb * 16 * (int)orow, dv_out);
          }
        }
      }
      if (out_lines) {
        u32x4_t ol[4];
        const rsrc_t rk = lines_rsrc(dKh[0], t0, n_end, orow);
        unstage_lines(stk, lane, ol);
#pragma unroll
        for (int j = 0; j < 4; ++j) store16_nt(rk, oline_off + j * 8 * (int)orow, ol[j]);
        const rsrc_t rv = lines_rsrc(dVh[0], t0, n_end, orow);
        unstage_lines(stv, lane, ol);
#pragma unroll
        for (int j = 0; j < 4; ++j) store16_nt(rv, oline_off + j * 8 * (int)orow, ol[j]);
      }
    }
  }
}

// Query pass of the backward for head-paired views.  A workgroup of eight
// waves takes heads 2u and 2u + 1 of one split: waves 2p and 2p + 1 (pair p)
// take heads 2u and 2u + 1 of the same 32-token tiles, 4k + p for k = 0, 1,
// ...  Per tile, the pair's first wave loads the 32 whole lines of Q (both
// heads) and the second those of dO into the pair's LDS tiles; after a
// barrier each wave computes its own head exactly as bwd_query_bf16 does, and
// dQ goes back through a line tile when the output pairs heads too.  Pair p
// sees the tiles of the one-head kernel's wave p, in the same order, so the
// partial dS and dz sum in the same order and the results are bit-identical to
// it.  Every wave runs the same number of tiles (those past the split's end
// load zeros and store nothing), as the loop holds workgroup barriers.
template <int ROPE>
__global__ __launch_bounds__(2 * kThreads) void bwd_query_bf16_lines(const u32x4_t* __restrict__ Q,
                                                                 const u32x4_t* __restrict__ dO,
                                                                 u32x4_t* __restrict__ dQ, Layout lin, Layout lout,
                                                                 StateView fwd, float eps, Rope rp, StateArgs a,
                                                                 int64_t units) {
  // line tiles: per pair Q, dO and dQ; then, after the loop, the reduction
  constexpr int kLines = 4 * 3 * kLineTile;
  constexpr int kRed = 2 * 4 * kStateElems;
  __shared__ __attribute__((aligned(16))) float smem[kLines > kRed ? kLines : kRed];
  __shared__ float tiles[8][ROPE ? 2 : 1][kTileFloats];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, 2 * kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  int64_t u, n_begin, n_end;
  int c, s;
  state_item(a, u, c, s, n_begin, n_end, units);
  const int64_t bh0 = 2 * u;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = w >> 1, hd = w & 1;
  const int64_t bh = bh0 + hd;
  const int n = lane & 15;
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only
  const int64_t irow = lin.token * 2, orow = lout.token * 2;  // bytes between tokens
  const int line_off = (lane >> 3) * (int)irow + (lane & 7) * 16;
  const int oline_off = (lane >> 3) * (int)orow + (lane & 7) * 16;
  const int out_off = n * (int)orow + g * 16;
  const int tab_off = n * 64 + g * 16;
  const bool out_lines = lout.head == kD;
  // the pair's first wave streams Q, the second dO
  const char* src = reinterpret_cast<const char*>(hd ? dO : Q) + lin.base(bh0) * 2;
  char* dQp = reinterpret_cast<char*>(dQ) + lout.base(bh0) * 2;
  char* dQh = reinterpret_cast<char*>(dQ) + lout.base(bh) * 2;
  float* st_q = smem + pr * 3 * kLineTile;
  float* st_o = st_q + kLineTile;
  float* st_dq = st_o + kLineTile;
  float* dn_tile = tiles[w][0];
  float* pq_tile = tiles[w][ROPE ? 1 : 0];

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
  for (int e = 0; e < 8; ++e) dzacc[e] = 0.f;

  // tile index i of the split -> tokens n_begin + 32 i; pair pr takes i = 4k + pr
  const int64_t n_tiles = (n_end - n_begin + 31) / 32;
  const int64_t iters = (n_tiles + 3) / 4;
  auto tile_t0 = [&](int64_t it) { return n_begin + 32 * (4 * it + pr); };
  u32x4_t nl[4];
  TileAnglesRows na;
  auto load_tile = [&](int64_t t0) {
    load_lines(lines_rsrc(src, t0, n_end, irow), line_off, irow, nl);
    if constexpr (ROPE == kRopeTable) load_angle_rows(rp.cos, rp.sin, rp.pos0, t0, n_end, tab_off, na);
  };
  if (iters > 0) load_tile(tile_t0(0));

  for (int64_t it = 0; it < iters; ++it) {
    const int64_t t0 = tile_t0(it);
    stage_lines(hd ? st_o : st_q, lane, nl);
    TileAnglesRows ang = na;
    __syncthreads();  // both halves of the pair's tile are staged
    if (it + 1 < iters) load_tile(tile_t0(it + 1));
    u32x4_t qx[2], ox[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      qx[tb] = staged_piece(st_q, tb, hd, n, g);
      ox[tb] = staged_piece(st_o, tb, hd, n, g);
    }
    const rsrc_t rdq = rows_rsrc(dQh, t0, n_end, orow);
    bf16x8_t bq[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const u32x4_t qr = relu_bf16x8(qx[tb]);
      bq[tb] = __builtin_bit_cast(bf16x8_t, qr);
      f32x4_t ang_c = ang.c[tb], ang_s = ang.s[tb];
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
      mfma3(srow, __builtin_bit_cast(bf16x8_t, ox[tb]), s0, s1);
      float gd[8], num[8], dr[8];
      unpack8(ox[tb], gd);
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
      if (out_lines)
        put_piece(st_dq, tb, hd, n, g, pack8(dr));
      else
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
    __syncthreads();  // the dQ tile is complete; every read of the Q and dO tiles is done
    if (out_lines) {
      u32x4_t x[4];
      unstage_lines(st_dq, lane, x);
      const rsrc_t r = lines_rsrc(dQp, t0, n_end, orow);
#pragma unroll
      for (int j = 2 * hd; j < 2 * hd + 2; ++j) store16_nt(r, oline_off + j * 8 * (int)orow, x[j]);
    }
  }

  // dz: sum the 16 lanes of each group (token rows), feature 8g + j
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = dzacc[e];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    dzacc[e] = x;
  }
  // partials of head hd: red[hd][pr] (the one-head kernel's wave pr)
  __syncthreads();  // the reduction area overlaps the line tiles
  float(*red)[4][kStateElems] = reinterpret_cast<float(*)[4][kStateElems]>(smem);
  float* rw = red[hd][pr];
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
    for (int e = 0; e < 8; ++e) rw[1024 + 8 * g + e] = dzacc[e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * kStateElems; idx += 2 * kThreads) {
    float(*r)[kStateElems] = red[idx / kStateElems];
    const int e = idx % kStateElems;
    r[0][e] = (r[0][e] + r[1][e]) + (r[2][e] + r[3][e]);
  }
  __syncthreads();
  // waves 0-3 write head 2u's partial, waves 4-7 head 2u + 1's
  write_partial(red[threadIdx.x >> 8][0], bh0 + (threadIdx.x >> 8), c, s, a, threadIdx.x & 255);
}

}  // namespace la
