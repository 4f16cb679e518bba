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
// The angles come from a table of the block's 256 tokens x 16 pairs that the
// workgroup writes, once per block, into the LDS stage the GEMM left free.
//
// Tiles of the (token range, head group) grid are dealt to the XCDs in
// contiguous runs, and inside a run walk 4 token ranges per head group: the
// workgroups resident on one XCD then share each x slice among several head
// groups and each weight slice among 4 token ranges in its L2.  The tiles of
// each XCD's last round, when few, run as halves or quarters (fewer heads, or
// fewer tokens on the query side), so that round fills more of the XCD.
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
  uint32_t G;       // tiles: M * Hp
};

// Tiles and the tail.  The grid holds G tiles (token range or block, head
// group).  The hardware deals workgroup blk to XCD blk % 8, and each XCD runs
// its workgroups in order, one per CU on its 32 CUs; XCD x takes a contiguous
// run of `count` tiles.  Equal tiles then run in rounds of 32, the last holding
// tail = count % 32.  That round runs with most CUs idle, so its tiles are cut
// into s parts each (s = 4 when the parts still fit on the 32 CUs at once,
// else 2, else none): the round then takes a part's time instead of a whole
// tile's.  Either way every (token, head) belongs to exactly one workgroup.
constexpr uint32_t kXcdCUs = 32;  // compute units per XCD

// parts per tail tile for a run of `count` tiles
__host__ __device__ inline uint32_t proj_parts(uint32_t count) {
  const uint32_t tail = count % kXcdCUs;
  return tail == 0 ? 1u : (4 * tail <= kXcdCUs ? 4u : (2 * tail <= kXcdCUs ? 2u : 1u));
}

// slots (workgroups) a run of `count` tiles takes
__host__ __device__ inline uint32_t proj_slots(uint32_t count) {
  return count + (proj_parts(count) - 1) * (count % kXcdCUs);
}

// Workgroups to launch for G tiles: every XCD gets as many slots as the
// busiest one needs (runs of G / 8 or G / 8 + 1 tiles); the spare slots exit
// at once.
__host__ __device__ inline uint32_t proj_grid(uint32_t G) {
  const uint32_t q = G / kXcds;
  uint32_t most = proj_slots(q);
  if (G % kXcds) {
    const uint32_t m1 = proj_slots(q + 1);
    most = m1 > most ? m1 : most;
  }
  return most * kXcds;
}

struct ProjTile {
  int64_t mi;  // token range (or block) row of the grid
  int pi;      // head group
  int parts;   // 1: the whole tile; 2, 4: one of that many parts
  int part;    // which one
};

// The tile of workgroup blk; false for a spare slot.  Inside an XCD's run the
// tiles walk kProjGroupM token ranges per head group, so the workgroups
// resident on one XCD share each x slice among head groups and each weight
// slice among token ranges in its L2.
__device__ __forceinline__ bool proj_tile(uint32_t blk, uint32_t G, int64_t M, int P, ProjTile* t) {
  const uint32_t q = G / kXcds, rem = G % kXcds, xcd = blk % kXcds, slot = blk / kXcds;
  const uint32_t count = q + (xcd < rem ? 1u : 0u), start = xcd * q + (xcd < rem ? xcd : rem);
  const uint32_t parts = proj_parts(count), whole = parts > 1 ? count - count % kXcdCUs : count;
  if (slot >= proj_slots(count)) return false;
  uint32_t L;
  if (slot < whole) {
    L = start + slot;
    t->parts = 1;
    t->part = 0;
  } else {
    L = start + whole + (slot - whole) / parts;
    t->parts = (int)parts;
    t->part = (int)((slot - whole) % parts);
  }
  const int64_t per_group = (int64_t)kProjGroupM * P;
  const int64_t first = ((int64_t)L / per_group) * kProjGroupM;
  const int64_t gsize = M - first < kProjGroupM ? M - first : kProjGroupM;
  const int64_t in = (int64_t)L % per_group;
  t->mi = first + in % gsize;
  t->pi = (int)(in / gsize);
  return true;
}

// Loads x and weight rows straight into LDS (buffer_load ... lds): a wave's
// instruction fills 1 KB of LDS, 16 rows of 64 bytes (one 32-channel step),
// lane l writing row l / 4, slot l % 4.  Slots are XOR-swizzled: slot s of row
// r holds 16-byte piece s ^ swz(r) of the row.  An MFMA operand read takes
// piece g of 16 consecutive rows in each quarter-wave; with swz(r) =
// ((r >> 2) ^ (r >> 1)) & 3 such a read runs at the LDS's full rate, 1 KB in
// about 4.6 cycles per CU, at every row offset the kernels use.  That was
// measured with 16-byte reads of each layout from 8 waves per CU: the layouts
// that simple bank models call conflict-free (no swizzle, or (r >> 1) ^ (r >>
// 3), or r >> 2, or r & 3) all take 8 cycles per 1 KB, half the rate.
__device__ __forceinline__ int proj_swz(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }

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

// The GEMM of one block of 256 (or 128) tokens: acc[i][j] (lane (n, g): tokens
// a_row + 16 i + 4 g + (0..3), column 16 j + n of this wave's 64; RB row
// blocks) over all nk 32-channel steps.  Three LDS stages of one step each (A:
// up to 256 token rows at 0, B: up to 256 weight rows at kProjBOff, 64 bytes a
// row).  Wave w's loads fill A rows 16 NA w .. + 16 NA - 1 (a_voff: row offsets
// in x, rsrc rx) and, for the first BW waves, B rows 16 NB w .. + 16 NB - 1
// (b_voff, rsrc rw); step k + 2 is loaded while step k computes.  Step t
// computes on stage t % 3.  Its barrier waits for the step's own loads (every
// wave's) to land and for step t - 1's reads to end everywhere; then stage
// (t + 2) % 3 is free for step t + 2's loads.  A wave issues NA + NB loads a
// step (NA when it stages no B rows), so with step t + 1's loads still in
// flight the wait is vmcnt(NA + NB) (vmcnt(NA) when only some waves stage B:
// the loads land in order, so the B-staging waves then also wait for one load
// of step t + 1, which has had a whole step to land), and vmcnt(0) at the last
// step.  In the main loop the stages are named, not indexed: the compiler then
// sees that the operand reads and the loads in flight touch different LDS
// arrays and adds no wait of its own, except at the loop head, where it cannot
// tell the stages apart across the back edge and waits for every load.  Six
// steps per iteration halve those waits (measured 3-4% faster than three; 24
// steps were no faster).  The caller has synchronised the workgroup since the
// stages were last read.
constexpr int kProjStage = (kProjTokens + kProjCols) * 64;  // bytes per stage
constexpr int kProjBOff = kProjTokens * 64;            // B rows after the A rows

template <int RB, int NA, int NB, int BW>
__device__ __forceinline__ void proj_gemm(rsrc_t rx, rsrc_t rw, const int (&a_voff)[NA], const int (&b_voff)[NB],
                                          int a_rd, int b_rd, int nk, int w, char* st0, char* st1, char* st2,
                                          f32x4_t (&acc)[RB][4]) {
  constexpr int kLoads = BW == kProjWaves ? NA + NB : NA;  // the wait count (see above)
  auto issue = [&](int k, char* stage) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_dma16(rx, stage + (16 * NA * w + 16 * i) * 64, a_voff[i] + k * 64);
    if (BW == kProjWaves || w < BW) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        lds_dma16(rw, stage + kProjBOff + (16 * NB * w + 16 * i) * 64, b_voff[i] + k * 64);
    }
  };
  auto compute = [&](const char* stage) {
    bf16x8_t bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const bf16x8_t*>(stage + b_rd + j * 1024);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(stage + a_rd + i * 1024);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af, bf[j], acc[i][j]);
    }
  };
  issue(0, st0);
  if (nk > 1) issue(1, st1);
  // steps k .. k + 2 (stages 0, 1, 2), every one with loads to issue
  auto three = [&](int k) {
    proj_stage_barrier<kLoads>();
    issue(k + 2, st2);
    compute(st0);
    proj_stage_barrier<kLoads>();
    issue(k + 3, st0);
    compute(st1);
    proj_stage_barrier<kLoads>();
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
      proj_stage_barrier<kLoads>();
    else
      proj_stage_barrier<0>();
    if (k + 2 < nk) issue(k + 2, nxt);
    compute(cur);
  }
}

// RoPE in the epilogues: once the GEMM of a block is done, its workgroup writes
// the cos/sin of every (token, pair) of the block into an LDS stage that no load
// or operand read touches any more (below), and the epilogue reads them from
// there.  Thread (token j = tid % 256, half = tid / 256) fills pairs
// 8 half .. 8 half + 7 of token j: its coordinates once, then four duos.
//
// Duo i of the half row: {cos, cos, sin, sin} of pairs 8 half + 2i and
// 8 half + 2i + 1 at position pos0 + tok (tok clamped into the call's tokens by
// the caller), from the per-axis tables staged in LDS (rtab) or the full
// tables in memory.
template <int ROPE>
__device__ __forceinline__ void proj_rope_half_row(const Rope& r, const float* rtab, int64_t tok, int half,
                                                   f32x4_t (&duo)[4]) {
  const int64_t pos = r.pos0 + tok;
  if constexpr (ROPE == kRopeAxes) {
    int t, h, w;
    rope_coords(r, pos, t, h, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) duo[i] = axis_duo(rtab, axis_entry(axis_pair(r, 8 * half + 2 * i), t, h, w));
  } else {
    const float* c = r.cos + pos * 16 + 8 * half;
    const float* s = r.sin + pos * 16 + 8 * half;
#pragma unroll
    for (int i = 0; i < 4; ++i) duo[i] = f32x4_t{c[2 * i], c[2 * i + 1], s[2 * i], s[2 * i + 1]};
  }
}

// The stage that the block's GEMM of nk steps leaves free: step k reads stage
// k % 3 and step k's loads were issued at step k - 2, so stage nk % 3 was last
// read at step nk - 3 and takes no load after it; every wave's reads of it ended
// before the barrier of step nk - 2.  A wave that has passed the last step's
// barrier may write it.
__device__ __forceinline__ char* proj_free_stage(int nk, char* st0, char* st1, char* st2) {
  const int s = nk % 3;
  return s == 0 ? st0 : (s == 1 ? st1 : st2);
}

// Hides a thread index from the compiler, so that the table writers' addresses
// are computed where they are used, after the GEMM.  Left visible, they are
// loop invariants that the compiler computes once ahead of the block loop and
// keeps live through the GEMM: at the register limit that costs the GEMM its
// operand prefetch (measured: 256 VGPRs and an MFMA stalled on each LDS read,
// about 5% slower tiles, against 233 VGPRs with the reads issued ahead).
__device__ __forceinline__ void opaque_index(int& i) { asm volatile("" : "+v"(i)); }

// Key/value epilogue table, pair-major: entry (pair q, token quad u) is 32
// bytes, cos of tokens 4u .. 4u+3 then their sin, at q * 2048 + (u ^ (q & 7)) *
// 32.  An epilogue read takes one pair's quad per lane; the XOR puts the eight
// pairs that a quarter-wave reads in distinct banks.  32 KB: one stage.
__device__ __forceinline__ int kv_tab_entry(int q, int u) { return q * 2048 + ((u ^ (q & 7)) << 5); }

template <int ROPE>
__device__ __forceinline__ void kv_rope_table(const Rope& r, const float* rtab, int64_t tok0, int64_t N, int tid,
                                              char* tab) {
  opaque_index(tid);
  const int j = tid & (kProjTokens - 1), half = tid / kProjTokens;
  const int64_t tok = tok0 + j < N ? tok0 + j : N - 1;
  f32x4_t duo[4];
  proj_rope_half_row<ROPE>(r, rtab, tok, half, duo);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float* p = reinterpret_cast<float*>(tab + kv_tab_entry(8 * half + 2 * i + e, j >> 2)) + (j & 3);
      p[0] = duo[i][e];
      p[4] = duo[i][2 + e];
    }
}

// Query epilogue table, token-major: token j's row is 128 bytes, duo d (pairs
// 2d, 2d + 1 as {cos, cos, sin, sin}) in 16-byte slot d ^ (j & 7) ^ ((j >> 3) &
// 1).  A read takes one duo of sixteen consecutive tokens (a lane each); the
// slot pattern keeps every eight of them (and every sixteen, with 64 banks)
// in distinct banks.  32 KB: one stage.
__device__ __forceinline__ int q_tab_entry(int j, int d) { return j * 128 + ((d ^ (j & 7) ^ ((j >> 3) & 1)) << 4); }

template <int ROPE>
__device__ __forceinline__ void q_rope_table(const Rope& r, const float* rtab, int64_t tok0, int64_t N, int tid,
                                             char* tab) {
  opaque_index(tid);
  const int j = tid & (kProjTokens - 1), half = tid / kProjTokens;
  const int64_t tok = tok0 + j < N ? tok0 + j : N - 1;
  f32x4_t duo[4];
  proj_rope_half_row<ROPE>(r, rtab, tok, half, duo);
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4_t*>(tab + q_tab_entry(j, 4 * half + i)) = duo[i];
}

// One tile: a token range of 256-token blocks and HG heads from head h (four;
// two for a half tile, one for a quarter), 8 waves.  Wave w takes head h + w /
// WPH and tokens TPW (w % WPH) .. + TPW - 1 of each block (WPH = 8 / HG waves
// per head, TPW = 256 / WPH tokens: 128, 64 or 32), 64 output columns (the
// head's key and value features: RB x 4 MFMA blocks of 16 x 16) through
// proj_gemm.  B row R of a stage is row R % 32 of head h + R / 64's key (bit 5
// of R clear) or value weights: 64 HG rows, 16 NB rows a wave (one head's 64
// rows fill only four waves' loads).  One workgroup fills a CU (96 KB of LDS,
// 104 KB with the per-axis RoPE tables).
template <int ROPE, int HG>
__device__ __forceinline__ void project_state_tile(const ProjArgs& p, const Rope& rp, const StateArgs& a, int64_t mi,
                                                   int h, char* st0, char* st1, char* st2, const float* rtab) {
  constexpr int WPH = 8 / HG;               // waves per head
  constexpr int TPW = kProjTokens / WPH;    // tokens per wave and block
  constexpr int RB = TPW / 16;              // its 16-token row blocks
  constexpr int NB = HG > 1 ? HG / 2 : 1;   // B loads (16 rows) per wave and step
  constexpr int BW = HG > 1 ? kProjWaves : 4;  // waves that stage B rows
  const int64_t b = mi / p.R;
  const int r = (int)(mi % p.R);
  const int64_t bh = b * p.H + h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int tw = w % WPH, hh = w / WPH;
  const int row = p.C * 2;  // bytes per token row and per weight row

  // loads: lane l fills row l / 4 (of 16), slot l % 4, with the swizzled piece
  const int dr = lane >> 2;
  const int dpiece = ((lane & 3) ^ proj_swz(dr)) * 16;
  int a_voff[2], b_voff[NB];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_voff[i] = (32 * w + 16 * i + dr) * row + dpiece;
  // wave w stages B rows rb0 .. rb0 + 16 NB - 1, all of one head and one matrix
  const int rb0 = 16 * NB * w;
#pragma unroll
  for (int i = 0; i < NB; ++i) b_voff[i] = ((rb0 >> 6) * 32 + ((rb0 + 16 * i) & 31) + dr) * row + dpiece;
  const int heads_here = p.H - h < HG ? p.H - h : HG;
  const rsrc_t rw =
      make_rsrc(((rb0 >> 5) & 1 ? p.wv : p.wk) + (int64_t)h * 32 * row, (int64_t)heads_here * 32 * row);
  const char* xb = p.x + b * p.N * (int64_t)row;
  // operand reads: lane (n, g) reads piece g of row base + n
  const int sw = 16 * (g ^ proj_swz(n));
  const int a_rd = (TPW * tw + n) * 64 + sw;
  const int b_rd = kProjBOff + (64 * hh + n) * 64 + sw;
  // RoPE: the pair partner's sign bits (flipped for even features), and where
  // this lane's angle quads sit in the block's table: pair 8 fh + (n >> 1),
  // token quad TPW / 4 tw + 8 t + 4 hs + g at tb[hs] + 16384 fh + 256 t
  const unsigned sgn_bits = (n & 1) ? 0u : 0x80008000u;
  int tb[2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) tb[hs] = kv_tab_entry(n >> 1, TPW / 4 * tw + 4 * hs + g);

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
    f32x4_t acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = zero4;
    __syncthreads();  // every wave is done with the previous block's stages
    proj_gemm<RB, 2, NB, BW>(rx, rw, a_voff, b_voff, a_rd, b_rd, nk, w, st0, st1, st2, acc);
    [[maybe_unused]] char* const tab = proj_free_stage(nk, st0, st1, st2);
    if constexpr (ROPE != kRopeNone) {
      kv_rope_table<ROPE>(rp, rtab, tok0, p.N, tid, tab);
      __syncthreads();  // the table is whole before any lane reads it
    }

    // acc[i][j], lane (n, g): tokens TPW tw + 16 i + 4 g + (0..3) of the
    // block, column 16 j + n of head h + hh (j = 0, 1: key features; 2, 3:
    // value features).  Row blocks 2t, 2t + 1 make one 32-token contraction.
#pragma unroll
    for (int t = 0; t < RB / 2; ++t) {
      bf16x8_t ka[2], vb[2];
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        ka[fh] = __builtin_bit_cast(bf16x8_t, pack_turned_relu(acc[2 * t][fh], acc[2 * t + 1][fh]));
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
        // tok0 + TPW tw + 16 (2t + s / 4) + 4 g + s % 4; the pair partner
        // f ^ 1 sits in lane n ^ 1, same slot.  Rotated: x c - x' s for even
        // f, x' s + x c for odd f, in fp32, then split into three bf16 parts
        // contracted against V one by one.  The partner comes over by DPP
        // with its sign already applied (an exact flip of the bf16 sign
        // bits); the angles of slots 4 hs .. 4 hs + 3 are one 16-byte quad of
        // cosines and one of sines.
        u32x4_t kw[2], pw[2];
#pragma unroll
        for (int fh = 0; fh < 2; ++fh) {
          kw[fh] = __builtin_bit_cast(u32x4_t, ka[fh]);
#pragma unroll
          for (int d = 0; d < 4; ++d)
            pw[fh][d] = (unsigned)__builtin_amdgcn_mov_dpp((int)kw[fh][d], 0xB1, 0xF, 0xF, false) ^ sgn_bits;
        }
        f32x4_t cq[2][2], sq[2][2];
#pragma unroll
        for (int fh = 0; fh < 2; ++fh)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const char* e = tab + tb[hs] + 16384 * fh + 256 * t;
            cq[fh][hs] = *reinterpret_cast<const f32x4_t*>(e);
            sq[fh][hs] = *reinterpret_cast<const f32x4_t*>(e + 16);
          }
        unsigned part[2][3][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float y[2][2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int slot = 2 * d + e;
#pragma unroll
            for (int fh = 0; fh < 2; ++fh) {
              const float x = e ? bf16hi_to_f32(kw[fh][d]) : bf16lo_to_f32(kw[fh][d]);
              const float xp = e ? bf16hi_to_f32(pw[fh][d]) : bf16lo_to_f32(pw[fh][d]);
              const float c = cq[fh][slot >> 2][slot & 3], sn = sq[fh][slot >> 2][slot & 3];
              y[fh][e] = __builtin_fmaf(x, c, xp * sn);  // the fusion fixed, as in rot_lo
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

  // The waves' sums to LDS, over stages 0 and 1 (no load is in flight after
  // the last step): wave (tw, hh) writes slot tw HG + hh, slots 0 .. 3 in
  // stage 0 and 4 .. 7 in stage 1, one state (kStateElems floats) each.  Then
  // head hq's sum, its token parts added in order, is written as partial r.
  __syncthreads();
  float* red0 = reinterpret_cast<float*>(st0);
  float* red1 = reinterpret_cast<float*>(st1);
  const int slot = tw * HG + hh;
  float* mine = (slot < 4 ? red0 : red1) + (slot & 3) * kStateElems;
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
  // element idx of head hq (idx < HG kStateElems) sits at idx + tw HG
  // kStateElems of the two stages taken as one run of 8 states
  for (int idx = tid; idx < HG * kStateElems; idx += kProjThreads) {
    float sum = red0[idx];
#pragma unroll
    for (int k = 1; k < WPH; ++k) {
      const int q = idx + k * HG * kStateElems;
      sum += q < 4 * kStateElems ? red0[q] : red1[q - 4 * kStateElems];
    }
    red0[idx] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < (HG + 1) / 2; ++j) {
    const int hq = 2 * j + (tid >> 8);
    if (hq < heads_here) write_partial(red0 + hq * kStateElems, bh + hq, 0, r, a, tid & 255);
  }
}

// Workgroup blk's tile (see proj_tile): a whole head group of four, or in an
// XCD's last round one of its halves (two heads) or quarters (one head).
template <int ROPE>
__global__ __launch_bounds__(kProjThreads, 1) void project_state_bf16(ProjArgs p, Rope rp, StateArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st1[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st2[kProjStage];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];

  ProjTile t;
  if (!proj_tile(blockIdx.x, p.G, p.M, p.Hp, &t)) return;
  const int h = 4 * t.pi + t.part * (4 / t.parts);
  if (h >= p.H) return;  // a part past the group's last head
  // the axis tables go to LDS; the first block's barrier orders the copy
  // before any lookup
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kProjThreads);
  if (t.parts == 1)
    project_state_tile<ROPE, 4>(p, rp, a, t.mi, h, st0, st1, st2, rtab);
  else if (t.parts == 2)
    project_state_tile<ROPE, 2>(p, rp, a, t.mi, h, st0, st1, st2, rtab);
  else
    project_state_tile<ROPE, 1>(p, rp, a, t.mi, h, st0, st1, st2, rtab);
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
  uint32_t G;        // tiles: M * Hq
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

// One tile: TT tokens from tok_off of a 256-token block and HG heads from head
// h (all 256 tokens and eight heads; four heads for a half tile; 128 tokens
// and four heads for a quarter), 8 waves.  Wave w takes heads h + 2 hh,
// h + 2 hh + 1 (hh = w / WPG) and tokens TPW tw .. + TPW - 1 of the tile
// (tw = w % WPG; WPG = 16 / HG waves per head pair, TPW = TT / WPG tokens:
// 128, 64 or 32).
template <int ROPE, int HG, int TT>
__device__ __forceinline__ void project_apply_tile(const ProjApplyArgs& p, const Rope& rp, int64_t mi, int tok_off,
                                                   int h, char* st0, char* st1, char* st2, const float* rtab) {
  constexpr int WPG = 16 / HG;             // waves per head pair
  constexpr int TPW = TT / WPG;            // tokens per wave
  constexpr int RB = TPW / 16;             // its 16-token row blocks
  constexpr int NA = TT / 128;             // A loads (16 rows) per wave and step
  constexpr int NB = HG / 4;               // B loads (16 rows) per wave and step
  const int64_t b = mi / p.R;
  const int64_t tok0 = (mi % p.R) * kProjTokens + tok_off;
  if (tok0 >= p.N) return;  // a quarter past the end of a ragged last block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int tw = w % WPG, hh = w / WPG;
  const int row = p.C * 2;

  const int dr = lane >> 2;
  const int dpiece = ((lane & 3) ^ proj_swz(dr)) * 16;
  int a_voff[NA], b_voff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) a_voff[i] = (16 * NA * w + 16 * i + dr) * row + dpiece;
  // wave w stages B rows 16 NB w .. + 16 NB - 1 (the query weights are 32 rows
  // a head, head-major)
#pragma unroll
  for (int i = 0; i < NB; ++i) b_voff[i] = (16 * NB * w + 16 * i + dr) * row + dpiece;
  const int heads_here = p.H - h < HG ? p.H - h : HG;
  const rsrc_t rw = make_rsrc(p.wq + (int64_t)h * 32 * row, (int64_t)heads_here * 32 * row);
  // rows at or past N read as zero; their outputs are not stored
  const rsrc_t rx = make_rsrc(p.x + (b * p.N + tok0) * (int64_t)row, (p.N - tok0) * row);
  const int sw = 16 * (g ^ proj_swz(n));
  const int a_rd = (TPW * tw + n) * 64 + sw;
  const int b_rd = kProjBOff + (64 * hh + n) * 64 + sw;
  // RoPE: this lane's pairs are 2g, 2g + 1, 8 + 2g, 9 + 2g (its k-slot pairs),
  // duos g and 4 + g of its token's row in the block's table (tokens
  // TPW tw + 16 m + n, m = 2t + bb: at tb[d] + 2048 m)
  int tb[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) tb[d] = q_tab_entry(TPW * tw + n, 4 * d + g);

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[RB][4];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4;
  __syncthreads();  // the RoPE tables are staged
  proj_gemm<RB, NA, NB, kProjWaves>(rx, rw, a_voff, b_voff, a_rd, b_rd, p.C / 32, w, st0, st1, st2, acc);
  [[maybe_unused]] char* const tab = proj_free_stage(p.C / 32, st0, st1, st2);
  if constexpr (ROPE != kRopeNone) {
    q_rope_table<ROPE>(rp, rtab, tok0, p.N, tid, tab);
    __syncthreads();  // the table is whole before any lane reads it
  }

  // acc[i][2u + fh], lane (n, g): tokens TPW tw + 16 i + 4 g + (0..3),
  // feature 16 fh + n of head h + 2 hh + u
  const bf16x8_t sel[2] = {untangle_select(g, n, 0), untangle_select(g, n, 1)};
  const int64_t tw0 = tok0 + TPW * tw;
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
    for (int t = 0; t < RB / 2; ++t) {
      bf16x8_t A[2];
#pragma unroll
      for (int fh = 0; fh < 2; ++fh)
        A[fh] = __builtin_bit_cast(bf16x8_t, pack_turned_relu(acc[2 * t][2 * u + fh], acc[2 * t + 1][2 * u + fh]));
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const f32x4_t d0 = mfma16(A[0], sel[bb], zero4), d1 = mfma16(A[1], sel[bb], zero4);
        const u32x4_t q = pack_turned_words(d0, d1);
        const int tr = 16 * (2 * t + bb) + n;  // this lane's token row in the wave's TPW
        f32x4_t c = zero4, sn = zero4;
        if constexpr (ROPE != kRopeNone) {
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const f32x4_t e = *reinterpret_cast<const f32x4_t*>(tab + tb[d] + 2048 * (2 * t + bb));
            c[2 * d] = e[0];
            c[2 * d + 1] = e[1];
            sn[2 * d] = e[2];
            sn[2 * d + 1] = e[3];
          }
        }
        store16_nt(ro, tr * (int)orow + 16 * g, apply_tile<ROPE != kRopeNone>(q, op, p.eps, c, sn));
      }
    }
  }
}

// Workgroup blk's tile (see proj_tile): a 256-token block and a group of eight
// heads, or in an XCD's last round one half of the group (four heads) or one
// quarter (four heads, 128 tokens: part 2 hq + th, heads 4 hq.., tokens
// 128 th..).
template <int ROPE>
__global__ __launch_bounds__(kProjThreads, 1) void project_apply_bf16(ProjApplyArgs p, Rope rp) {
  __shared__ __attribute__((aligned(1024))) char st0[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st1[kProjStage];
  __shared__ __attribute__((aligned(1024))) char st2[kProjStage];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];

  ProjTile t;
  if (!proj_tile(blockIdx.x, p.G, p.M, p.Hq, &t)) return;
  const int hq = t.parts == 4 ? t.part >> 1 : t.part;  // which four heads (parts 2 and 4)
  const int h = 8 * t.pi + (t.parts == 1 ? 0 : 4 * hq);
  if (h >= p.H) return;  // a part past the group's last head
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kProjThreads);
  if (t.parts == 1)
    project_apply_tile<ROPE, 8, 256>(p, rp, t.mi, 0, h, st0, st1, st2, rtab);
  else if (t.parts == 2)
    project_apply_tile<ROPE, 4, 256>(p, rp, t.mi, 0, h, st0, st1, st2, rtab);
  else
    project_apply_tile<ROPE, 4, 128>(p, rp, t.mi, 128 * (t.part & 1), h, st0, st1, st2, rtab);
}

}  // namespace la
