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

}  // namespace la
