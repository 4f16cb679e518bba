// Host side of the C ABI declared in include/sana_linattn.h: argument checks,
// launch geometry, workspace layout and the 3D RoPE table builder.
//
// Every compute call works on heads of N tokens split into C chunks of L
// tokens (C = 1 for all calls but block_causal) and enqueues up to three
// kernels on the caller's stream:
//   1. state pass  (Pc workgroups per chunk, each a contiguous token range,
//                   writing one partial state; with one chunk and one split
//                   the workgroup writes the head's state itself)
//   2. finalize    (when there are several partials: one thread per state
//                   element walks a head's partials in order from the carried
//                   state, storing the running sum at every chunk end and
//                   committing the last)
//   3. apply pass  (equal contiguous ranges of the flattened head x token
//                   space, one per workgroup, each cut at head and chunk
//                   boundaries)
// state_update runs 1-2 only, apply runs 3 only.  The backward runs 1-2 to
// recompute the chunk states (backward_saved reads those the forward left in
// the workspace), then its query pass, a reverse finalize and its key pass.
// Views whose heads 2u, 2u + 1 share 128-byte lines (bf16, H even) run the
// passes per head pair, reading whole lines (la_lines.h).  RoPE comes as full
// cos/sin tables or as per-axis tables; each kernel is instantiated for none,
// either form.  Nothing is allocated, freed or synchronised.

#include "sana_linattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <atomic>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "la_backward.h"
#include "la_conv.h"
#include "la_kernels.h"
#include "la_lines.h"
#include "la_proj.h"

// sha256[:16] of the kernel sources, passed in by the build
#ifndef SANA_SOURCE_HASH
#define SANA_SOURCE_HASH "unknown"
#endif

// Scratch of sana_linattn_block_forward_noalloc: one copy per GPU.  In host
// code this name is a stand-in, not a device address; host code uses only the
// address that scratch_address() looks up.
static __device__ __align__(256) unsigned char scratch[SANA_NOALLOC_SCRATCH_BYTES];

namespace {

// MI355X: 256 compute units.  Both passes size their grids to one resident
// round of workgroups, at the count that measured fastest: state 2 per CU (8
// waves, each with a 64-token chunk of K and V in flight; the RoPE variant's
// register use allows no more), apply 3 per CU on the Sana-1.6B 4096 px layer
// (4 were slower there), and 4 per CU with RoPE on the 720p layer, where each
// wave computes longer per chunk and more waves keep more loads in flight.
constexpr int64_t kCUs = 256;
constexpr int64_t kStateGroups = kCUs * 2;
constexpr int64_t kApplyGroups = kCUs * 3;
constexpr int64_t kApplyGroupsRope = kCUs * 4;
constexpr int64_t kMaxSplits = 64;       // partial states per chunk
constexpr int64_t kMinSplitTokens = 256;
// With at least this many (head, chunk) items of at most kWholeChunkTokens
// tokens, one workgroup per chunk beats splitting; with one chunk the state
// pass then writes the states itself and the finalize launch (~3.5 us) is
// skipped.
constexpr int64_t kWholeChunkItems = kCUs / 2;
constexpr int64_t kWholeChunkTokens = 1024;
constexpr int64_t kMinApplyTokens = 256;
constexpr int64_t kMinApplyTokensF32 = 256;
constexpr int64_t kMaxApplyTokensF32 = 1024;
// a launch may hold at most 2^32 - 1 work-items: 2^24 - 1 workgroups of 256
constexpr int64_t kMaxGroups = ((int64_t)1 << 24) - 1;
// Apply with the finalize folded in: at most this many CUs' worth of
// workgroups per head (each workgroup reads the head's partials), and heads of
// at most this many tokens.
constexpr int64_t kFoldMaxParts = 4;
constexpr int64_t kFoldMaxTokens = 1 << 20;
// heads longer than this take 8-wave folded-apply workgroups, shorter 16-wave
constexpr int64_t kFoldWideTokens = 8192;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

struct Geometry {
  int64_t BH = 0, N = 0, L = 0, C = 0;
  int64_t Pc = 0, Ls = 0;  // state pass: splits per chunk, tokens per split
  int64_t Ga = 0, La = 0;  // bf16 apply pass: workgroups, flattened tokens per workgroup
  int64_t T = 0, Lt = 0;   // fp32 apply pass: tiles per chunk, tokens per tile
  size_t partial_off = 0, state_off = 0, total_bytes = 0;
};

// Heads of N tokens in chunks of L (L >= N: one chunk).
Geometry make_geometry(int64_t BH, int64_t N, int64_t L, bool rope) {
  Geometry g;
  g.BH = BH;
  g.N = N;
  if (BH <= 0 || N <= 0) return g;
  g.L = L < N ? L : N;
  g.C = ceil_div(N, g.L);
  // splits per chunk: about kStateGroups workgroups in all, at least
  // kMinSplitTokens tokens each (none for many short chunks)
  int64_t p = ceil_div(kStateGroups / BH, g.C);
  if (BH * g.C >= kWholeChunkItems && g.L <= kWholeChunkTokens) p = 1;
  const int64_t p_max = ceil_div(g.L, kMinSplitTokens);
  if (p > p_max) p = p_max;
  if (p > kMaxSplits) p = kMaxSplits;
  if (p < 1) p = 1;
  g.Ls = round_up(ceil_div(g.L, p), 32);
  g.Pc = ceil_div(g.L, g.Ls);

  const int64_t total = BH * N;
  int64_t la = round_up(ceil_div(total, rope ? kApplyGroupsRope : kApplyGroups), 64);
  if (la < kMinApplyTokens) la = kMinApplyTokens;
  if (ceil_div(total, la) > kMaxGroups) la = round_up(ceil_div(total, kMaxGroups), 64);
  g.La = la;
  g.Ga = ceil_div(total, la);

  int64_t lt = round_up(ceil_div(g.L, ceil_div(kApplyGroups, BH * g.C)), 64);
  if (lt < kMinApplyTokensF32) lt = kMinApplyTokensF32;
  if (lt > kMaxApplyTokensF32) lt = kMaxApplyTokensF32;
  const int64_t per = kMaxGroups / (BH * g.C);
  if (per >= 1) {
    const int64_t lt_floor = round_up(ceil_div(g.L, per), 64);
    if (lt < lt_floor) lt = lt_floor;
  }
  g.Lt = lt;
  g.T = ceil_div(g.L, lt);

  const int64_t state = (int64_t)la::kStateElems * (int64_t)sizeof(float);
  // (+ one word per head and part: the arrival flags of apply_fold_bf16)
  const int64_t partials = g.C * g.Pc > 1 ? BH * g.C * g.Pc * state + BH * kFoldMaxParts * 16 * 4 : 0;
  g.partial_off = 0;
  g.state_off = (size_t)round_up(partials, 256);
  g.total_bytes = g.state_off + (size_t)round_up(BH * g.C * state, 256);
  return g;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

int elem_size(int dtype) { return dtype == SANA_DT_BF16 ? 2 : (dtype == SANA_DT_F32 ? 4 : 0); }

// Checks shared by every compute call.  Returns SANA_OK and fills `elems`
// (B*H*N*D) and `BH` when the sizes are valid.
int check_sizes(int B, int H, int64_t N, int D, int dtype, int64_t* BH, int64_t* elems) {
  if (B < 0 || H < 0 || N < 0 || D <= 0) return SANA_ERR_INVALID;
  if (elem_size(dtype) == 0) return SANA_ERR_INVALID;
  if (D != la::kD) return SANA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)B * (int64_t)H;
  if (bh > 0 && N > (INT64_MAX / 64) / bh) return SANA_ERR_INVALID;
  if (bh > kMaxGroups) return SANA_ERR_INVALID;
  *BH = bh;
  *elems = bh * N * D;
  return SANA_OK;
}

// A RoPE argument in the per-axis form names a latent grid.
bool axis_form(const sana_rope* rope) { return rope->grid[0] != 0 || rope->grid[1] != 0 || rope->grid[2] != 0; }

int check_rope(const sana_rope* rope, int64_t N) {
  if (!rope) return SANA_OK;
  if (!rope->cos || !rope->sin) return SANA_ERR_INVALID;
  if (rope->pos_offset < 0 || rope->n_pos < 0) return SANA_ERR_INVALID;
  if (rope->pos_offset > rope->n_pos || N > rope->n_pos - rope->pos_offset) return SANA_ERR_INVALID;
  if (!axis_form(rope)) {
    if (rope->pairs[0] || rope->pairs[1] || rope->pairs[2]) return SANA_ERR_INVALID;
    return aligned(rope->cos, 16) && aligned(rope->sin, 16) ? SANA_OK : SANA_ERR_INVALID;
  }
  // per-axis tables: positions are the grid's points, the pairs split the
  // head's 16 in even counts, the tables fit the kernels' LDS copy, and the coordinates of a
  // position come out exact (grid plane below 2^20 points, positions below 2^31)
  const int64_t T = rope->grid[0], Hl = rope->grid[1], Wl = rope->grid[2];
  const int64_t pt = rope->pairs[0], ph = rope->pairs[1], pw = rope->pairs[2];
  if (T <= 0 || Hl <= 0 || Wl <= 0 || pt < 0 || ph < 0 || pw < 0 || pt + ph + pw != la::kD / 2)
    return SANA_ERR_INVALID;
  if (pt % 2 || ph % 2) return SANA_ERR_INVALID;  // pairs (2i, 2i+1) share an axis
  if (Hl * Wl >= ((int64_t)1 << 20) || T * Hl * Wl >= ((int64_t)1 << 31) || rope->n_pos != T * Hl * Wl)
    return SANA_ERR_INVALID;
  if (T * pt + Hl * ph + Wl * pw > la::kMaxAxisTab) return SANA_ERR_INVALID;
  return aligned(rope->cos, 4) && aligned(rope->sin, 4) ? SANA_OK : SANA_ERR_INVALID;
}

// Grid bounds of the state pass and the fp32 apply pass.
bool grids_fit(const Geometry& g) { return g.BH * g.C * g.Pc <= kMaxGroups && g.BH * g.C * g.T <= kMaxGroups; }

int check_workspace(const Geometry& g, const void* ws, size_t ws_bytes) {
  if (!grids_fit(g)) return SANA_ERR_INVALID;
  if (!ws || ws_bytes < g.total_bytes) return SANA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SANA_ERR_INVALID;
  return SANA_OK;
}

int check_tensor(const void* p) { return (p && aligned(p, 16)) ? SANA_OK : SANA_ERR_INVALID; }

// An address span [p, p + bytes) a call reads or writes.
struct Span {
  const void* p;
  size_t bytes;
};

// Bytes of the RoPE tables a call reads (none without RoPE).
size_t rope_table_bytes(const sana_rope* rope) {
  if (!rope) return 0;
  if (rope->grid[0] || rope->grid[1] || rope->grid[2])
    return (size_t)((int64_t)rope->grid[0] * rope->pairs[0] + (int64_t)rope->grid[1] * rope->pairs[1] +
                    (int64_t)rope->grid[2] * rope->pairs[2]) * sizeof(float);
  return (size_t)rope->n_pos * (la::kD / 2) * sizeof(float);
}

// The part of the workspace a call writes may overlap none of the tensors,
// states or tables it touches.
int check_workspace_overlaps(const void* ws, size_t used, std::initializer_list<Span> spans,
                             const sana_rope* rope) {
  for (const Span& t : spans)
    if (overlaps(ws, used, t.p, t.bytes)) return SANA_ERR_INVALID;
  if (rope) {
    const size_t tab = rope_table_bytes(rope);
    if (overlaps(ws, used, rope->cos, tab) || overlaps(ws, used, rope->sin, tab)) return SANA_ERR_INVALID;
  }
  return SANA_OK;
}

// A tensor's element layout and the bytes from its first element to one past
// its last.
struct View {
  la::Layout lay;
  size_t span = 0;
};

// Strides (stride, extent) nested without overlap: sorted by stride, each
// stride at least the span of everything inside it (a row is D elements).
bool injective(int64_t D, const int64_t (&stride)[3], const int64_t (&extent)[3]) {
  int order[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (stride[order[j]] < stride[order[i]]) {
        const int t = order[i];
        order[i] = order[j];
        order[j] = t;
      }
  int64_t inner = D;
  for (int i = 0; i < 3; ++i) {
    const int a = order[i];
    if (extent[a] <= 1) continue;
    if (stride[a] < inner) return false;
    inner = stride[a] * (extent[a] - 1) + inner;
  }
  return true;
}

// The view of a [B][H][N][D] tensor through `l` (NULL: contiguous).  Rows
// (token starts) must be 16-byte aligned and at least D elements apart; the
// bf16 kernels address a 64-token window with 32-bit offsets, so a row stride
// is limited to 16 MiB.  Outputs must not map two elements to one address.
int make_view(const sana_layout* l, int B, int H, int64_t N, int D, int es, bool output, View* v) {
  if (!l) {
    v->lay = la::Layout{(int64_t)H * N * D, N * D, D, H};
  } else {
    if (l->batch < 0 || l->head < 0 || l->token < D) return SANA_ERR_INVALID;
    if ((l->batch * es) % 16 || (l->head * es) % 16 || (l->token * es) % 16) return SANA_ERR_INVALID;
    if (l->token * es > ((int64_t)1 << 24)) return SANA_ERR_INVALID;
    if (l->batch > (INT64_MAX / 4) / (B > 0 ? B : 1) || l->head > (INT64_MAX / 4) / (H > 0 ? H : 1) ||
        l->token > (INT64_MAX / 4) / (N > 0 ? N : 1))
      return SANA_ERR_INVALID;
    if (output) {
      const int64_t stride[3] = {l->batch, l->head, l->token}, extent[3] = {B, H, N};
      if (!injective(D, stride, extent)) return SANA_ERR_INVALID;
    }
    v->lay = la::Layout{l->batch, l->head, l->token, H};
  }
  if (B > 0 && H > 0 && N > 0)
    v->span = (size_t)(((int64_t)(B - 1) * v->lay.batch + (int64_t)(H - 1) * v->lay.head +
                        (N - 1) * v->lay.token + D) * es);
  return SANA_OK;
}

// q/k/v/o against one another and against the state buffers: o may not
// overlap anything; among the states only exact in-place aliasing
// (kv_out == kv_in, ksum_out == ksum_in) is allowed.
int check_overlaps(const void* q, const void* k, const void* v, const void* o, size_t in_span, size_t out_span,
                   const float* kv_in, const float* ksum_in, const float* kv_out, const float* ksum_out, int64_t bh) {
  if (overlaps(o, out_span, q, in_span) || overlaps(o, out_span, k, in_span) || overlaps(o, out_span, v, in_span))
    return SANA_ERR_INVALID;
  const size_t kv_bytes = (size_t)bh * 1024 * sizeof(float), ks_bytes = (size_t)bh * 32 * sizeof(float);
  const void* tensors[4] = {q, k, v, o};
  const size_t spans[4] = {in_span, in_span, in_span, out_span};
  const void* states[4] = {kv_in, ksum_in, kv_out, ksum_out};
  const size_t state_sizes[4] = {kv_bytes, ks_bytes, kv_bytes, ks_bytes};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      if (overlaps(states[i], state_sizes[i], tensors[j], spans[j])) return SANA_ERR_INVALID;
  if (overlaps(kv_in, kv_bytes, ksum_in, ks_bytes) || overlaps(kv_out, kv_bytes, ksum_out, ks_bytes) ||
      overlaps(kv_in, kv_bytes, ksum_out, ks_bytes) || overlaps(ksum_in, ks_bytes, kv_out, kv_bytes))
    return SANA_ERR_INVALID;
  if (kv_out && overlaps(kv_in, kv_bytes, kv_out, kv_bytes) && kv_in != kv_out) return SANA_ERR_INVALID;
  if (ksum_out && overlaps(ksum_in, ks_bytes, ksum_out, ks_bytes) && ksum_in != ksum_out) return SANA_ERR_INVALID;
  return SANA_OK;
}

la::StateArgs state_args(void* ws, const Geometry& g, const float* kv_in, const float* ksum_in, float* kv_out,
                         float* ksum_out) {
  la::StateArgs a;
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + g.partial_off);
  a.states = reinterpret_cast<float*>(static_cast<char*>(ws) + g.state_off);
  a.kv_in = kv_in;
  a.ksum_in = ksum_in;
  a.kv_out = kv_out;
  a.ksum_out = ksum_out;
  a.N = g.N;
  a.L = g.L;
  a.Ls = g.Ls;
  a.C = (int)g.C;
  a.Pc = (int)g.Pc;
  return a;
}

// The workspace's per-chunk states (33 x 32 layout), as the apply pass reads them.
la::StateView ws_view(const la::StateArgs& a) {
  return la::StateView{a.states, a.states + 1024, la::kStateElems, la::kStateElems};
}

// Whether adjacent heads of one token are adjacent 64-byte rows, so that one
// 128-byte line holds two heads: the bf16 passes then give each workgroup two
// heads of the same tokens.
bool paired_heads(const la::Layout& l) { return l.head == la::kD; }

// Pairs (2u, 2u + 1) that never straddle two batches can be read as whole
// lines by one wave (la_lines.h).
bool whole_lines(const la::Layout& l) { return paired_heads(l) && l.H % 2 == 0; }

// The kernels' view of a call's RoPE argument: its form (la::kRopeNone,
// kRopeTable or kRopeAxes) and the angle source.  N: tokens in the call.
struct RopeArg {
  int kind = la::kRopeNone;
  la::Rope r{};
};

RopeArg rope_arg(const sana_rope* rope, int64_t N) {
  RopeArg a;
  if (!rope) return a;
  a.r.cos = rope->cos;
  a.r.sin = rope->sin;
  a.r.pos0 = rope->pos_offset;
  a.r.pos_last = rope->pos_offset + (N > 0 ? N - 1 : 0);
  if (!axis_form(rope)) {
    a.kind = la::kRopeTable;
    return a;
  }
  a.kind = la::kRopeAxes;
  const int T = rope->grid[0], Hl = rope->grid[1], Wl = rope->grid[2];
  a.r.Hl = Hl;
  a.r.Wl = Wl;
  a.r.pt = rope->pairs[0];
  a.r.ph = rope->pairs[1];
  a.r.base_h = T * rope->pairs[0];
  a.r.base_w = a.r.base_h + Hl * rope->pairs[1];
  a.r.n_tab = a.r.base_w + Wl * rope->pairs[2];
  a.r.inv_w = 1.0 / Wl;
  a.r.inv_hw = 1.0 / ((double)Hl * Wl);
  return a;
}

// Calls f(std::integral_constant<int, kind>) for the RoPE form `kind`, so a
// launch site names each kernel once for all three forms.
template <typename F>
void with_rope(int kind, F&& f) {
  if (kind == la::kRopeAxes)
    f(std::integral_constant<int, la::kRopeAxes>{});
  else if (kind == la::kRopeTable)
    f(std::integral_constant<int, la::kRopeTable>{});
  else
    f(std::integral_constant<int, la::kRopeNone>{});
}

// The ordered sum of every head's C x Pc partials into its chunk states
// (reverse: the suffix sums of the backward pass), one thread per state
// element, with 16 partials in flight per thread, or 64 when a head has more
// than 16.
void launch_finalize(const la::StateArgs& a, int64_t BH, hipStream_t st, bool reverse = false) {
  const int64_t n_elems = BH * la::kStateElems;
  const dim3 grid((unsigned)ceil_div(n_elems, la::kThreads)), block(la::kThreads);
  const bool deep = a.C * a.Pc > 16;
  if (reverse) {
    if (deep)
      la::state_finalize_reverse<64><<<grid, block, 0, st>>>(a, n_elems);
    else
      la::state_finalize_reverse<16><<<grid, block, 0, st>>>(a, n_elems);
  } else {
    if (deep)
      la::state_finalize<64><<<grid, block, 0, st>>>(a, n_elems);
    else
      la::state_finalize<16><<<grid, block, 0, st>>>(a, n_elems);
  }
}

// State pass, and the finalize when there are several partials per head.
void launch_state(const void* k, const void* v, const la::Layout& lkv, int dtype, const Geometry& g,
                  const RopeArg& ra, const la::StateArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(g.BH * g.C * g.Pc)), block(la::kThreads);
  with_rope(ra.kind, [&](auto R) {
    constexpr int RO = decltype(R)::value;
    if (dtype == SANA_DT_BF16) {
      const la::u32x4_t* K = static_cast<const la::u32x4_t*>(k);
      const la::u32x4_t* V = static_cast<const la::u32x4_t*>(v);
      const dim3 pgrid((unsigned)(ceil_div(g.BH, 2) * g.C * g.Pc)), pblock(2 * la::kThreads);
      if (lkv.token == la::kD)
        la::state_bf16<RO, true, 1><<<grid, block, 0, st>>>(K, V, lkv, ra.r, a, g.BH);
      else if (whole_lines(lkv))
        la::state_bf16_lines<RO><<<pgrid, block, 0, st>>>(K, V, lkv, ra.r, a, g.BH / 2);
      else if (paired_heads(lkv))
        la::state_bf16<RO, false, 2><<<pgrid, pblock, 0, st>>>(K, V, lkv, ra.r, a, g.BH);
      else
        la::state_bf16<RO, false, 1><<<grid, block, 0, st>>>(K, V, lkv, ra.r, a, g.BH);
    } else {
      la::state_f32<RO><<<grid, block, 0, st>>>(static_cast<const float*>(k), static_cast<const float*>(v), lkv,
                                                ra.r, a);
    }
  });
  if (g.C * g.Pc > 1) launch_finalize(a, g.BH, st);
}

void launch_apply(const void* q, void* o, const la::Layout& lq, const la::Layout& lo, int dtype, float eps,
                  const Geometry& g, const RopeArg& ra, const la::StateView& sv, hipStream_t st) {
  with_rope(ra.kind, [&](auto R) {
    constexpr int RO = decltype(R)::value;
    if (dtype == SANA_DT_BF16) {
      const la::u32x4_t* Q = static_cast<const la::u32x4_t*>(q);
      la::u32x4_t* O = static_cast<la::u32x4_t*>(o);
      const bool dense = lq.token == la::kD && lo.token == la::kD;
      const bool lines = !dense && whole_lines(lq);
      const bool pair = !dense && (paired_heads(lq) || paired_heads(lo));
      // ranges of g.La tokens over (head, token), or per head pair
      const int64_t units = pair ? ceil_div(g.BH, 2) : g.BH;
      const dim3 grid((unsigned)(pair ? units * ceil_div(g.N, g.La) : ceil_div(units * g.N, g.La))),
          block(pair && !lines ? 2 * la::kThreads : la::kThreads);
      if (lines)
        la::apply_bf16_lines<RO><<<grid, block, 0, st>>>(Q, O, lq, lo, sv, g.N, g.L, (int)g.C, g.La, eps, ra.r, units);
      else if (dense)
        la::apply_bf16<RO, true, 1><<<grid, block, 0, st>>>(Q, O, lq, lo, sv, g.N, g.L, (int)g.C, units * g.N, g.La,
                                                            eps, ra.r, g.BH);
      else if (pair)
        la::apply_bf16<RO, false, 2><<<grid, block, 0, st>>>(Q, O, lq, lo, sv, g.N, g.L, (int)g.C, units * g.N, g.La,
                                                             eps, ra.r, g.BH);
      else
        la::apply_bf16<RO, false, 1><<<grid, block, 0, st>>>(Q, O, lq, lo, sv, g.N, g.L, (int)g.C, units * g.N, g.La,
                                                             eps, ra.r, g.BH);
    } else {
      const dim3 grid((unsigned)(g.BH * g.C * g.T)), block(la::kThreads);
      la::apply_f32<RO><<<grid, block, 0, st>>>(static_cast<const float*>(q), static_cast<float*>(o), lq, lo, sv, g.N,
                                                g.L, (int)g.C, (int)g.T, g.Lt, eps, ra.r);
    }
  });
}

int launch_status() { return hipGetLastError() == hipSuccess ? SANA_OK : SANA_ERR_HIP; }

// One launch per call (forward_whole_bf16): each head one chunk of one split,
// dense bf16 layouts, no full-table RoPE.
bool whole_head(int dtype, const Geometry& g, bool dense, int rope_kind) {
  return dtype == SANA_DT_BF16 && g.C == 1 && g.Pc == 1 && dense && rope_kind != la::kRopeTable;
}

// Waves per workgroup of the folded apply.  Each workgroup reads its head's
// partials once, so chunk-sized heads take one 16-wave workgroup per CU (fewer
// copies of the partials against few bytes per head), longer heads two 8-wave
// workgroups per CU (every CU busy; measured 3% faster on 16384 tokens, 1.6%
// slower on 4680).
int fold_waves(const Geometry& g) { return g.N > kFoldWideTokens ? 8 : 16; }

// Workgroups per head of the apply with the finalize folded in
// (apply_fold_bf16), or 0 where the three-launch path is taken.  It needs one
// chunk in 2 .. kFoldMaxSplits splits, dense bf16 layouts and no full-table RoPE; a
// head's P workgroups share one XCD's 32 CUs with the XCD's other heads, and
// together they keep at least half the CUs busy.
int64_t fold_parts(int dtype, const Geometry& g, bool dense, int rope_kind) {
  if (dtype != SANA_DT_BF16 || g.C != 1 || g.Pc < 2 || g.Pc > la::kFoldMaxSplits || !dense ||
      rope_kind == la::kRopeTable || g.N > kFoldMaxTokens)
    return 0;
  // 16 waves resident per CU
  const int64_t per_cu = 16 / fold_waves(g);
  int64_t P = (kCUs / la::kXcdCount) * per_cu / ceil_div(g.BH, la::kXcdCount);
  if (P > kFoldMaxParts * per_cu) P = kFoldMaxParts * per_cu;
  if (P < 2 || g.BH * P < kCUs * per_cu / 2) return 0;
  return P;
}

// A fresh number per folded call: its commit over a carried state waits for
// flags holding this call's number (see apply_fold_bf16).
std::atomic<unsigned> g_fold_epoch{0x5a5a0001u};

// State pass (items dealt XCD by XCD), then the apply that sums the partials.
template <int RO>
void launch_fold(const void* q, const void* k, const void* v, void* o, const la::Layout& lin, const la::Layout& lo,
                 const Geometry& g, int64_t P, const RopeArg& ra, const la::StateArgs& a, float eps, hipStream_t st) {
  const int64_t heads_per_xcd = ceil_div(g.BH, la::kXcdCount);
  la::state_bf16<RO, true, 1, true><<<dim3((unsigned)(la::kXcdCount * heads_per_xcd * g.Pc)), dim3(la::kThreads), 0, st>>>(
      static_cast<const la::u32x4_t*>(k), static_cast<const la::u32x4_t*>(v), lin, ra.r, a, g.BH);
  la::FoldArgs f;
  f.P = (int)P;
  f.Na = round_up(ceil_div(g.N, P), 64);
  // the flags live in the partials' scratch past the partials themselves
  f.flags = (a.kv_out && a.kv_in) ? reinterpret_cast<unsigned*>(a.partials + g.BH * g.Pc * la::kStateElems) : nullptr;
  f.epoch = g_fold_epoch.fetch_add(2u, std::memory_order_relaxed);
  const dim3 grid((unsigned)(la::kXcdCount * heads_per_xcd * P));
  const auto* Q = static_cast<const la::u32x4_t*>(q);
  auto* O = static_cast<la::u32x4_t*>(o);
  if (fold_waves(g) == 8)
    la::apply_fold_bf16<8, RO><<<grid, dim3(64 * 8), 0, st>>>(Q, O, lin, lo, a, f, g.BH, eps, ra.r);
  else
    la::apply_fold_bf16<16, RO><<<grid, dim3(64 * 16), 0, st>>>(Q, O, lin, lo, a, f, g.BH, eps, ra.r);
}

// Shared body of forward, block_forward and block_causal: chunks of L tokens
// (L >= N for one chunk), carried state in, optional commit out.
int attend(const void* q, const void* k, const void* v, void* o, const sana_layout* in, const sana_layout* out,
           const float* kv_in, const float* ksum_in, float* kv_out, float* ksum_out, int B, int H, int64_t N,
           int64_t L, int D, int dtype, float eps, const sana_rope* rope, void* ws, size_t ws_bytes,
           void* hip_stream) {
  int64_t bh = 0, elems = 0;
  int rc = check_sizes(B, H, N, D, dtype, &bh, &elems);
  if (rc != SANA_OK) return rc;
  if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID;
  if (L <= 0) return SANA_ERR_INVALID;
  if (elems == 0) return SANA_OK;
  if (check_tensor(q) || check_tensor(k) || check_tensor(v) || check_tensor(o)) return SANA_ERR_INVALID;
  if ((kv_in == nullptr) != (ksum_in == nullptr)) return SANA_ERR_INVALID;
  if ((kv_out == nullptr) != (ksum_out == nullptr)) return SANA_ERR_INVALID;
  if ((kv_in && (!aligned(kv_in, 4) || !aligned(ksum_in, 4))) ||
      (kv_out && (!aligned(kv_out, 4) || !aligned(ksum_out, 4))))
    return SANA_ERR_INVALID;
  View vin, vout;
  if ((rc = make_view(in, B, H, N, D, elem_size(dtype), false, &vin)) != SANA_OK) return rc;
  if ((rc = make_view(out, B, H, N, D, elem_size(dtype), true, &vout)) != SANA_OK) return rc;
  if ((rc = check_overlaps(q, k, v, o, vin.span, vout.span, kv_in, ksum_in, kv_out, ksum_out, bh)) != SANA_OK)
    return rc;
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  const Geometry g = make_geometry(bh, N, L, rope != nullptr);
  if ((rc = check_workspace(g, ws, ws_bytes)) != SANA_OK) return rc;
  {
    const size_t kv_bytes = (size_t)bh * 1024 * sizeof(float), ks_bytes = (size_t)bh * 32 * sizeof(float);
    if ((rc = check_workspace_overlaps(ws, g.total_bytes,
                                       {{q, vin.span}, {k, vin.span}, {v, vin.span}, {o, vout.span},
                                        {kv_in, kv_bytes}, {ksum_in, ks_bytes}, {kv_out, kv_bytes},
                                        {ksum_out, ks_bytes}},
                                       rope)) != SANA_OK)
      return rc;
  }

  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const la::StateArgs a = state_args(ws, g, kv_in, ksum_in, kv_out, ksum_out);
  const RopeArg ra = rope_arg(rope, N);
  // one chunk of one split per head, dense bf16 layouts: a head's state and
  // its apply in one workgroup, one launch (the full-table RoPE form keeps
  // the two passes)
  const bool dense = vin.lay.token == la::kD && vout.lay.token == la::kD;
  // one chunk split a few ways over a few dozen heads: the apply sums the
  // partials itself, two launches
  if (const int64_t P = fold_parts(dtype, g, dense, ra.kind)) {
    if (ra.kind == la::kRopeAxes)
      launch_fold<la::kRopeAxes>(q, k, v, o, vin.lay, vout.lay, g, P, ra, a, eps, st);
    else
      launch_fold<la::kRopeNone>(q, k, v, o, vin.lay, vout.lay, g, P, ra, a, eps, st);
    return launch_status();
  }
  if (whole_head(dtype, g, dense, ra.kind)) {
    with_rope(ra.kind, [&](auto R) {
      constexpr int RO = decltype(R)::value;
      if constexpr (RO != la::kRopeTable)
        la::forward_whole_bf16<RO><<<dim3((unsigned)g.BH), dim3(la::kThreads), 0, st>>>(
            static_cast<const la::u32x4_t*>(k), static_cast<const la::u32x4_t*>(v),
            static_cast<const la::u32x4_t*>(q), static_cast<la::u32x4_t*>(o), vin.lay, vout.lay, ra.r, a, N, eps);
    });
    return launch_status();
  }
  launch_state(k, v, vin.lay, dtype, g, ra, a, st);
  launch_apply(q, o, vin.lay, vout.lay, dtype, eps, g, ra, ws_view(a), st);
  return launch_status();
}

// Key pass of the backward: dK, dV from the state gradient G_c of every chunk.
void launch_key_pass(const void* k, const void* v, void* dk, void* dv, const la::Layout& lin,
                     const la::Layout& lout, int dtype, const Geometry& g, const RopeArg& ra,
                     const la::StateView& view, hipStream_t st) {
  const dim3 block(la::kThreads);
  with_rope(ra.kind, [&](auto R) {
    constexpr int RO = decltype(R)::value;
    if (dtype == SANA_DT_BF16) {
      const dim3 kgrid((unsigned)g.Ga);
      const auto* K = static_cast<const la::u32x4_t*>(k);
      const auto* V = static_cast<const la::u32x4_t*>(v);
      auto* dK = static_cast<la::u32x4_t*>(dk);
      auto* dV = static_cast<la::u32x4_t*>(dv);
      if (lin.token != la::kD && whole_lines(lin))
        la::bwd_key_bf16_lines<RO><<<dim3((unsigned)(g.BH / 2 * ceil_div(g.N, g.La))), block, 0, st>>>(
            K, V, dK, dV, lin, lout, view, g.N, g.L, (int)g.C, g.La, ra.r, g.BH / 2);
      else if (lin.token == la::kD && lout.token == la::kD)
        la::bwd_key_bf16<RO, true><<<kgrid, block, 0, st>>>(K, V, dK, dV, lin, lout, view, g.N, g.L, (int)g.C,
                                                            g.BH * g.N, g.La, ra.r);
      else
        la::bwd_key_bf16<RO, false><<<kgrid, block, 0, st>>>(K, V, dK, dV, lin, lout, view, g.N, g.L, (int)g.C,
                                                             g.BH * g.N, g.La, ra.r);
    } else {
      const dim3 kgrid((unsigned)(g.BH * g.C * g.T));
      la::bwd_key_vec<RO><<<kgrid, block, 0, st>>>(static_cast<const float*>(k), static_cast<const float*>(v),
                                                   static_cast<float*>(dk), static_cast<float*>(dv), lin, lout, view,
                                                   g.N, g.L, (int)g.C, (int)g.T, g.Lt, ra.r);
    }
  });
}

// Backward: recompute the chunk states (state pass + finalize), then the query
// pass (dQ, partial dS/dz), the reverse finalize (suffix sums G_c, gradient of
// the carried state) and the key pass (dK, dV).  The workspace layout is the
// forward's: the query pass reuses the partials, the reverse finalize
// overwrites the chunk states with G_c once the query pass has read them.
void launch_backward(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
                     const la::Layout& lin, const la::Layout& lout, int dtype, float eps, const Geometry& g,
                     const RopeArg& ra, const la::StateArgs& fwd, const la::StateArgs& bwd, hipStream_t st) {
  const la::StateView view = ws_view(fwd);
  const dim3 block(la::kThreads);
  const dim3 qgrid((unsigned)(g.BH * g.C * g.Pc));
  with_rope(ra.kind, [&](auto R) {
    constexpr int RO = decltype(R)::value;
    if (dtype == SANA_DT_BF16) {
      const auto* Q = static_cast<const la::u32x4_t*>(q);
      const auto* dO = static_cast<const la::u32x4_t*>(dout);
      auto* dQ = static_cast<la::u32x4_t*>(dq);
      const dim3 pgrid((unsigned)(ceil_div(g.BH, 2) * g.C * g.Pc));
      if (lin.token == la::kD && lout.token == la::kD)
        la::bwd_query_bf16<RO, true><<<qgrid, block, 0, st>>>(Q, dO, dQ, lin, lout, view, eps, ra.r, bwd);
      else if (whole_lines(lin))
        la::bwd_query_bf16_lines<RO><<<pgrid, dim3(2 * la::kThreads), 0, st>>>(Q, dO, dQ, lin, lout, view, eps, ra.r,
                                                                               bwd, g.BH / 2);
      else
        la::bwd_query_bf16<RO, false><<<qgrid, block, 0, st>>>(Q, dO, dQ, lin, lout, view, eps, ra.r, bwd);
    } else {
      la::bwd_query_vec<RO><<<qgrid, block, 0, st>>>(static_cast<const float*>(q), static_cast<const float*>(dout),
                                                     static_cast<float*>(dq), lin, lout, view, eps, ra.r, bwd);
    }
  });
  if (g.C * g.Pc > 1) launch_finalize(bwd, g.BH, st, true);
  launch_key_pass(k, v, dk, dv, lin, lout, dtype, g, ra, view, st);
}

bool state_pair_ok(const float* s, const float* z) {
  if ((s == nullptr) != (z == nullptr)) return false;
  return !s || (aligned(s, 4) && aligned(z, 4));
}

// saved: ws holds the chunk states of the forward call (no recompute).
int backward(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
             const sana_layout* in, const sana_layout* out, const float* kv_in, const float* ksum_in,
             const float* dkv_out, const float* dksum_out, float* dkv_in, float* dksum_in, int B, int H, int64_t N,
             int64_t L, int D, int dtype, float eps, const sana_rope* rope, void* ws, size_t ws_bytes,
             void* hip_stream, bool saved = false) {
  int64_t bh = 0, elems = 0;
  int rc = check_sizes(B, H, N, D, dtype, &bh, &elems);
  if (rc != SANA_OK) return rc;
  if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID;
  if (L <= 0) return SANA_ERR_INVALID;
  if (!state_pair_ok(kv_in, ksum_in) || !state_pair_ok(dkv_out, dksum_out) || !state_pair_ok(dkv_in, dksum_in))
    return SANA_ERR_INVALID;
  if (elems == 0) return SANA_OK;
  const void* inputs[4] = {q, k, v, dout};
  void* outputs[3] = {dq, dk, dv};
  for (const void* p : inputs)
    if (check_tensor(p)) return SANA_ERR_INVALID;
  for (void* p : outputs)
    if (check_tensor(p)) return SANA_ERR_INVALID;
  View vin, vout;
  if ((rc = make_view(in, B, H, N, D, elem_size(dtype), false, &vin)) != SANA_OK) return rc;
  if ((rc = make_view(out, B, H, N, D, elem_size(dtype), true, &vout)) != SANA_OK) return rc;
  const size_t ibytes = vin.span, obytes = vout.span;
  const size_t kv_bytes = (size_t)bh * 1024 * sizeof(float), ks_bytes = (size_t)bh * 32 * sizeof(float);
  // outputs overlap nothing; state gradients overlap no tensor, and dkv_in may
  // only alias dkv_out exactly (likewise the key sums)
  const void* states[6] = {kv_in, ksum_in, dkv_out, dksum_out, dkv_in, dksum_in};
  const size_t state_sizes[6] = {kv_bytes, ks_bytes, kv_bytes, ks_bytes, kv_bytes, ks_bytes};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outputs[i], obytes, inputs[j], ibytes)) return SANA_ERR_INVALID;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outputs[i], obytes, outputs[j], obytes)) return SANA_ERR_INVALID;
    for (int j = 0; j < 6; ++j)
      if (overlaps(outputs[i], obytes, states[j], state_sizes[j])) return SANA_ERR_INVALID;
  }
  for (int i = 0; i < 6; ++i)
    for (int j = 0; j < 4; ++j)
      if (overlaps(states[i], state_sizes[i], inputs[j], ibytes)) return SANA_ERR_INVALID;
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j) {
      if (!overlaps(states[i], state_sizes[i], states[j], state_sizes[j])) continue;
      const bool in_place = (i == 2 && j == 4 && states[i] == states[j]) || (i == 3 && j == 5 && states[i] == states[j]);
      if (!in_place) return SANA_ERR_INVALID;
    }
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  const Geometry g = make_geometry(bh, N, L, rope != nullptr);
  if ((rc = check_workspace(g, ws, ws_bytes)) != SANA_OK) return rc;
  if ((rc = check_workspace_overlaps(ws, g.total_bytes,
                                     {{q, ibytes}, {k, ibytes}, {v, ibytes}, {dout, ibytes}, {dq, obytes},
                                      {dk, obytes}, {dv, obytes}, {kv_in, kv_bytes}, {ksum_in, ks_bytes},
                                      {dkv_out, kv_bytes}, {dksum_out, ks_bytes}, {dkv_in, kv_bytes},
                                      {dksum_in, ks_bytes}},
                                     rope)) != SANA_OK)
    return rc;

  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const la::StateArgs fwd = state_args(ws, g, kv_in, ksum_in, nullptr, nullptr);
  const la::StateArgs bwd = state_args(ws, g, dkv_out, dksum_out, dkv_in, dksum_in);
  const RopeArg ra = rope_arg(rope, N);
  if (!saved) launch_state(k, v, vin.lay, dtype, g, ra, fwd, st);
  launch_backward(q, k, v, dout, dq, dk, dv, vin.lay, vout.lay, dtype, eps, g, ra, fwd, bwd, st);
  return launch_status();
}

size_t workspace(int B, int H, int64_t N, int64_t L, int D, int dtype, int has_rope) {
  int64_t bh = 0, elems = 0;
  if (L <= 0 || check_sizes(B, H, N, D, dtype, &bh, &elems) != SANA_OK) return 0;
  return make_geometry(bh, N, L, has_rope != 0).total_bytes;
}

// Fused K/V projection and state pass: each batch's token blocks of 256 are
// cut into R ranges of T blocks, one workgroup per (range, four heads), each
// range of a head leaving one partial state (none when R = 1: the workgroup
// writes the state itself).  At most kProjMaxRanges partials per head keep the
// finalize's reads small next to the GEMM.
constexpr int64_t kProjMaxRanges = 128;
constexpr int kProjMaxChannels = 65536;  // keeps the kernel's 32-bit byte offsets in range

struct ProjGeometry {
  int64_t BH = 0, R = 0, T = 0, G = 0;
  size_t state_off = 0, total_bytes = 0;
};

// Checks the sizes of sana_linattn_project_state and lays out its workspace.
int make_proj_geometry(int B, int H, int64_t N, int C, int D, int dtype, ProjGeometry* pg) {
  if (B < 0 || H < 0 || N < 0 || C <= 0 || D <= 0 || elem_size(dtype) == 0) return SANA_ERR_INVALID;
  if (D != la::kD || dtype != SANA_DT_BF16) return SANA_ERR_UNSUPPORTED;
  if (C % la::kProjChannelQuantum || C > kProjMaxChannels) return SANA_ERR_INVALID;
  const int64_t bh = (int64_t)B * H;
  if (bh > kMaxGroups || (B > 0 && N > (INT64_MAX / 4) / ((int64_t)B * C))) return SANA_ERR_INVALID;
  ProjGeometry g;
  g.BH = bh;
  if (bh > 0 && N > 0) {
    const int64_t nblk = ceil_div(N, la::kProjTokens);
    g.T = ceil_div(nblk, kProjMaxRanges);
    g.R = ceil_div(nblk, g.T);
    g.G = (int64_t)B * g.R * ceil_div(H, 4);
    if (g.G > kMaxGroups) return SANA_ERR_INVALID;
    const int64_t state = (int64_t)la::kStateElems * (int64_t)sizeof(float);
    g.state_off = (size_t)round_up(g.R > 1 ? bh * g.R * state : 0, 256);
    g.total_bytes = g.state_off + (size_t)round_up(bh * state, 256);
  }
  *pg = g;
  return SANA_OK;
}

// The device address of the current GPU's scratch array: looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SANA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SANA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SANA_OK;
}

}  // namespace

extern "C" {

size_t sana_linattn_workspace_bytes(int B, int H, int64_t N, int D, int dtype, int has_rope) {
  return workspace(B, H, N, N > 0 ? N : 1, D, dtype, has_rope);
}

size_t sana_linattn_block_causal_workspace_bytes(int B, int H, int64_t N, int64_t chunk, int D, int dtype,
                                                 int has_rope) {
  return workspace(B, H, N, chunk, D, dtype, has_rope);
}

int sana_linattn_forward_launches(int B, int H, int64_t N, int64_t chunk, int D, int dtype, int rope_form,
                                  int dense) {
  int64_t bh = 0, elems = 0;
  if (chunk <= 0 || rope_form < 0 || rope_form > 2 || check_sizes(B, H, N, D, dtype, &bh, &elems) != SANA_OK)
    return 0;
  if (elems == 0) return 0;
  const int kind = rope_form == 2 ? la::kRopeAxes : (rope_form == 1 ? la::kRopeTable : la::kRopeNone);
  const Geometry g = make_geometry(bh, N, chunk, rope_form != 0);
  if (whole_head(dtype, g, dense != 0, kind)) return 1;
  if (fold_parts(dtype, g, dense != 0, kind)) return 2;
  return g.C * g.Pc > 1 ? 3 : 2;
}

int sana_linattn_forward(const void* q, const void* k, const void* v, void* o, int B, int H, int64_t N, int D,
                         int dtype, float eps, const sana_rope* rope, void* ws, size_t ws_bytes,
                         void* hip_stream) {
  return attend(q, k, v, o, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, N, N > 0 ? N : 1, D, dtype,
                eps, rope, ws, ws_bytes, hip_stream);
}

int sana_linattn_forward_strided(const void* q, const void* k, const void* v, void* o, const sana_layout* in,
                                 const sana_layout* out, int B, int H, int64_t N, int D, int dtype, float eps,
                                 const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream) {
  return attend(q, k, v, o, in, out, nullptr, nullptr, nullptr, nullptr, B, H, N, N > 0 ? N : 1, D, dtype, eps,
                rope, ws, ws_bytes, hip_stream);
}

int sana_linattn_block_forward(const void* q, const void* k, const void* v, void* o, const float* kv_in,
                               const float* ksum_in, float* kv_out, float* ksum_out, int B, int H, int64_t N,
                               int D, int dtype, float eps, const sana_rope* rope, void* ws, size_t ws_bytes,
                               void* hip_stream) {
  return attend(q, k, v, o, nullptr, nullptr, kv_in, ksum_in, kv_out, ksum_out, B, H, N, N > 0 ? N : 1, D, dtype,
                eps, rope, ws, ws_bytes, hip_stream);
}

int sana_linattn_block_forward_noalloc(const void* q, const void* k, const void* v, void* o, const float* kv_in,
                                       const float* ksum_in, float* kv_out, float* ksum_out, int B, int H, int64_t N,
                                       int D, int dtype, float eps, const sana_rope* rope, void* hip_stream) {
  // too large for the array: rejected before any device call
  if (workspace(B, H, N, N > 0 ? N : 1, D, dtype, rope != nullptr) > SANA_NOALLOC_SCRATCH_BYTES)
    return SANA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != SANA_OK) return rc;
  return attend(q, k, v, o, nullptr, nullptr, kv_in, ksum_in, kv_out, ksum_out, B, H, N, N > 0 ? N : 1, D, dtype,
                eps, rope, ws, SANA_NOALLOC_SCRATCH_BYTES, hip_stream);
}

int sana_linattn_block_forward_strided(const void* q, const void* k, const void* v, void* o, const sana_layout* in,
                                       const sana_layout* out, const float* kv_in, const float* ksum_in,
                                       float* kv_out, float* ksum_out, int B, int H, int64_t N, int D, int dtype,
                                       float eps, const sana_rope* rope, void* ws, size_t ws_bytes,
                                       void* hip_stream) {
  return attend(q, k, v, o, in, out, kv_in, ksum_in, kv_out, ksum_out, B, H, N, N > 0 ? N : 1, D, dtype, eps, rope,
                ws, ws_bytes, hip_stream);
}

int sana_linattn_block_causal(const void* q, const void* k, const void* v, void* o, const float* kv_in,
                              const float* ksum_in, float* kv_out, float* ksum_out, int B, int H, int64_t N,
                              int64_t chunk, int D, int dtype, float eps, const sana_rope* rope, void* ws,
                              size_t ws_bytes, void* hip_stream) {
  return attend(q, k, v, o, nullptr, nullptr, kv_in, ksum_in, kv_out, ksum_out, B, H, N, chunk, D, dtype, eps, rope,
                ws, ws_bytes, hip_stream);
}

int sana_linattn_block_causal_strided(const void* q, const void* k, const void* v, void* o, const sana_layout* in,
                                      const sana_layout* out, const float* kv_in, const float* ksum_in,
                                      float* kv_out, float* ksum_out, int B, int H, int64_t N, int64_t chunk, int D,
                                      int dtype, float eps, const sana_rope* rope, void* ws, size_t ws_bytes,
                                      void* hip_stream) {
  return attend(q, k, v, o, in, out, kv_in, ksum_in, kv_out, ksum_out, B, H, N, chunk, D, dtype, eps, rope, ws,
                ws_bytes, hip_stream);
}

size_t sana_linattn_backward_workspace_bytes(int B, int H, int64_t N, int64_t chunk, int D, int dtype,
                                            int has_rope) {
  return workspace(B, H, N, chunk, D, dtype, has_rope);
}

int sana_linattn_backward(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                          void* dv, const float* kv_in, const float* ksum_in, const float* dkv_out,
                          const float* dksum_out, float* dkv_in, float* dksum_in, int B, int H, int64_t N,
                          int64_t chunk, int D, int dtype, float eps, const sana_rope* rope, void* ws,
                          size_t ws_bytes, void* hip_stream) {
  return backward(q, k, v, dout, dq, dk, dv, nullptr, nullptr, kv_in, ksum_in, dkv_out, dksum_out, dkv_in, dksum_in,
                  B, H, N, chunk, D, dtype, eps, rope, ws, ws_bytes, hip_stream);
}

int sana_linattn_backward_strided(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                                  void* dv, const sana_layout* in, const sana_layout* out, const float* kv_in,
                                  const float* ksum_in, const float* dkv_out, const float* dksum_out, float* dkv_in,
                                  float* dksum_in, int B, int H, int64_t N, int64_t chunk, int D, int dtype,
                                  float eps, const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream) {
  return backward(q, k, v, dout, dq, dk, dv, in, out, kv_in, ksum_in, dkv_out, dksum_out, dkv_in, dksum_in, B, H, N,
                  chunk, D, dtype, eps, rope, ws, ws_bytes, hip_stream);
}

int sana_linattn_backward_saved(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                                void* dv, const sana_layout* in, const sana_layout* out, const float* dkv_out,
                                const float* dksum_out, float* dkv_in, float* dksum_in, int B, int H, int64_t N,
                                int64_t chunk, int D, int dtype, float eps, const sana_rope* rope, void* ws,
                                size_t ws_bytes, void* hip_stream) {
  return backward(q, k, v, dout, dq, dk, dv, in, out, nullptr, nullptr, dkv_out, dksum_out, dkv_in, dksum_in, B, H, N,
                  chunk, D, dtype, eps, rope, ws, ws_bytes, hip_stream, true);
}

int sana_linattn_state_update_backward(const void* k, const void* v, const float* dkv, const float* dksum,
                                       void* dk, void* dv, int B, int H, int64_t N, int D, int dtype,
                                       const sana_rope* rope, void* hip_stream) {
  int64_t bh = 0, elems = 0;
  int rc = check_sizes(B, H, N, D, dtype, &bh, &elems);
  if (rc != SANA_OK) return rc;
  if (elems == 0) return SANA_OK;
  if (check_tensor(k) || check_tensor(v) || check_tensor(dk) || check_tensor(dv)) return SANA_ERR_INVALID;
  if (!dkv || !dksum || !aligned(dkv, 4) || !aligned(dksum, 4)) return SANA_ERR_INVALID;
  const size_t bytes = (size_t)elems * elem_size(dtype);
  const size_t kv_bytes = (size_t)bh * 1024 * sizeof(float), ks_bytes = (size_t)bh * 32 * sizeof(float);
  const void* ins[4] = {k, v, dkv, dksum};
  const size_t in_bytes[4] = {bytes, bytes, kv_bytes, ks_bytes};
  for (int i = 0; i < 4; ++i)
    if (overlaps(dk, bytes, ins[i], in_bytes[i]) || overlaps(dv, bytes, ins[i], in_bytes[i])) return SANA_ERR_INVALID;
  if (overlaps(dk, bytes, dv, bytes)) return SANA_ERR_INVALID;
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  const Geometry g = make_geometry(bh, N, N, rope != nullptr);
  if (!grids_fit(g)) return SANA_ERR_INVALID;
  const la::Layout flat{(int64_t)H * N * D, N * D, D, H};
  launch_key_pass(k, v, dk, dv, flat, flat, dtype, g, rope_arg(rope, N), la::StateView{dkv, dksum, 1024, 32},
                  static_cast<hipStream_t>(hip_stream));
  return launch_status();
}

int sana_linattn_state_update(const void* k, const void* v, float* kv_state, float* ksum_state, int B, int H,
                              int64_t N, int D, int dtype, const sana_rope* rope, void* ws, size_t ws_bytes,
                              void* hip_stream) {
  int64_t bh = 0, elems = 0;
  int rc = check_sizes(B, H, N, D, dtype, &bh, &elems);
  if (rc != SANA_OK) return rc;
  if (elems == 0) return SANA_OK;
  if (check_tensor(k) || check_tensor(v)) return SANA_ERR_INVALID;
  if (!kv_state || !ksum_state || !aligned(kv_state, 4) || !aligned(ksum_state, 4)) return SANA_ERR_INVALID;
  const size_t bytes = (size_t)elems * elem_size(dtype);
  const size_t kv_bytes = (size_t)bh * 1024 * sizeof(float), ks_bytes = (size_t)bh * 32 * sizeof(float);
  if (overlaps(kv_state, kv_bytes, ksum_state, ks_bytes) || overlaps(kv_state, kv_bytes, k, bytes) ||
      overlaps(kv_state, kv_bytes, v, bytes) || overlaps(ksum_state, ks_bytes, k, bytes) ||
      overlaps(ksum_state, ks_bytes, v, bytes))
    return SANA_ERR_INVALID;
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  const Geometry g = make_geometry(bh, N, N, rope != nullptr);
  if ((rc = check_workspace(g, ws, ws_bytes)) != SANA_OK) return rc;
  if ((rc = check_workspace_overlaps(ws, g.total_bytes,
                                     {{k, bytes}, {v, bytes}, {kv_state, kv_bytes}, {ksum_state, ks_bytes}},
                                     rope)) != SANA_OK)
    return rc;

  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const la::Layout flat{(int64_t)H * N * D, N * D, D, H};
  launch_state(k, v, flat, dtype, g, rope_arg(rope, N), state_args(ws, g, kv_state, ksum_state, kv_state, ksum_state),
               st);
  return launch_status();
}

int sana_linattn_apply(const void* q, void* o, const float* kv_state, const float* ksum_state, int B, int H,
                       int64_t N, int D, int dtype, float eps, const sana_rope* rope, void* hip_stream) {
  int64_t bh = 0, elems = 0;
  int rc = check_sizes(B, H, N, D, dtype, &bh, &elems);
  if (rc != SANA_OK) return rc;
  if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID;
  if (elems == 0) return SANA_OK;
  if (check_tensor(q) || check_tensor(o)) return SANA_ERR_INVALID;
  if (!kv_state || !ksum_state || !aligned(kv_state, 4) || !aligned(ksum_state, 4)) return SANA_ERR_INVALID;
  const size_t bytes = (size_t)elems * elem_size(dtype);
  const size_t kv_bytes = (size_t)bh * 1024 * sizeof(float), ks_bytes = (size_t)bh * 32 * sizeof(float);
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, kv_state, kv_bytes) || overlaps(o, bytes, ksum_state, ks_bytes))
    return SANA_ERR_INVALID;
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  const Geometry g = make_geometry(bh, N, N, rope != nullptr);
  if (!grids_fit(g)) return SANA_ERR_INVALID;
  const la::Layout flat{(int64_t)H * N * D, N * D, D, H};
  launch_apply(q, o, flat, flat, dtype, eps, g, rope_arg(rope, N), la::StateView{kv_state, ksum_state, 1024, 32},
               static_cast<hipStream_t>(hip_stream));
  return launch_status();
}

int sana_linattn_temporal_conv3(const void* x, void* y, const float* w, const float* bias, const void* cache_in,
                                void* cache_out, int B, int F, int64_t S, int C, int dtype, void* hip_stream) {
  const int es = elem_size(dtype);
  if (B < 0 || F < 0 || S < 0 || C < 0 || es == 0) return SANA_ERR_INVALID;
  if (C % 8) return SANA_ERR_INVALID;
  if (S > 0 && C > 0 && (int64_t)B > (INT64_MAX / 64) / S / C) return SANA_ERR_INVALID;
  const int64_t cols = (int64_t)B * S * (C / 8);
  if (cols == 0 || F == 0) return SANA_OK;
  if (S * (int64_t)C > (INT64_MAX / 64) / F) return SANA_ERR_INVALID;
  if (check_tensor(x) || check_tensor(y)) return SANA_ERR_INVALID;
  if (!w || !aligned(w, 16) || (bias && !aligned(bias, 16))) return SANA_ERR_INVALID;
  if ((cache_in && !aligned(cache_in, 16)) || (cache_out && !aligned(cache_out, 16))) return SANA_ERR_INVALID;
  const size_t bytes = (size_t)B * F * S * C * es, cbytes = (size_t)B * S * C * es;
  if (overlaps(y, bytes, x, bytes) || overlaps(y, bytes, cache_in, cbytes) || overlaps(y, bytes, cache_out, cbytes) ||
      overlaps(cache_out, cbytes, x, bytes))
    return SANA_ERR_INVALID;
  if (cache_out && overlaps(cache_out, cbytes, cache_in, cbytes) && cache_out != cache_in) return SANA_ERR_INVALID;
  if (overlaps(y, bytes, w, (size_t)C * 3 * sizeof(float)) || overlaps(y, bytes, bias, (size_t)C * sizeof(float)))
    return SANA_ERR_INVALID;
  const int64_t blocks = ceil_div(cols, la::kThreads);
  if (blocks > INT32_MAX) return SANA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (dtype == SANA_DT_BF16)
    la::temporal_conv3<__bf16><<<dim3((unsigned)blocks), dim3(la::kThreads), 0, st>>>(
        static_cast<const __bf16*>(x), static_cast<__bf16*>(y), w, bias, static_cast<const __bf16*>(cache_in),
        static_cast<__bf16*>(cache_out), F, S, C, cols);
  else
    la::temporal_conv3<float><<<dim3((unsigned)blocks), dim3(la::kThreads), 0, st>>>(
        static_cast<const float*>(x), static_cast<float*>(y), w, bias, static_cast<const float*>(cache_in),
        static_cast<float*>(cache_out), F, S, C, cols);
  return launch_status();
}

int sana_linattn_rope3d_table(int T, int Hl, int Wl, int D, int dt, int dh, int dw, double base, float* cos_host,
                              float* sin_host) {
  if (T < 0 || Hl < 0 || Wl < 0 || D <= 0 || dt < 0 || dh < 0 || dw < 0) return SANA_ERR_INVALID;
  if ((dt | dh | dw) & 1 || dt + dh + dw != D || !(base > 0.0) || !std::isfinite(base)) return SANA_ERR_INVALID;
  const int64_t n = (int64_t)T * Hl * Wl;
  if (n == 0) return SANA_OK;
  if (!cos_host || !sin_host) return SANA_ERR_INVALID;
  const int pairs = D / 2;
  const int widths[3] = {dt, dh, dw};
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < Hl; ++h)
      for (int w = 0; w < Wl; ++w) {
        const int64_t row = ((int64_t)t * Hl + h) * Wl + w;
        const double coord[3] = {(double)t, (double)h, (double)w};
        int p = 0;
        for (int a = 0; a < 3; ++a)
          for (int kk = 0; kk < widths[a] / 2; ++kk, ++p) {
            const double theta = coord[a] * std::pow(base, -2.0 * kk / widths[a]);
            cos_host[row * pairs + p] = (float)std::cos(theta);
            sin_host[row * pairs + p] = (float)std::sin(theta);
          }
      }
  return SANA_OK;
}

int sana_linattn_rope3d_axes(int T, int Hl, int Wl, int D, int dt, int dh, int dw, double base, float* cos_host,
                             float* sin_host) {
  if (T < 0 || Hl < 0 || Wl < 0 || D <= 0 || dt < 0 || dh < 0 || dw < 0) return SANA_ERR_INVALID;
  if ((dt | dh | dw) & 1 || dt + dh + dw != D || !(base > 0.0) || !std::isfinite(base)) return SANA_ERR_INVALID;
  const int extent[3] = {T, Hl, Wl};
  const int widths[3] = {dt, dh, dw};
  if ((int64_t)T * dt + (int64_t)Hl * dh + (int64_t)Wl * dw == 0) return SANA_OK;
  if (!cos_host || !sin_host) return SANA_ERR_INVALID;
  int64_t at = 0;
  for (int a = 0; a < 3; ++a)
    for (int x = 0; x < extent[a]; ++x)
      for (int kk = 0; kk < widths[a] / 2; ++kk, ++at) {
        // the same expression as the full tables' entry for this axis
        const double theta = (double)x * std::pow(base, -2.0 * kk / widths[a]);
        cos_host[at] = (float)std::cos(theta);
        sin_host[at] = (float)std::sin(theta);
      }
  return SANA_OK;
}

size_t sana_linattn_project_state_workspace_bytes(int B, int H, int64_t N, int C, int D, int dtype) {
  ProjGeometry g;
  return make_proj_geometry(B, H, N, C, D, dtype, &g) == SANA_OK ? g.total_bytes : 0;
}

int sana_linattn_project_state(const void* x, const void* w_k, const void* w_v, float* kv_state, float* ksum_state,
                               int B, int H, int64_t N, int C, int D, int dtype, const sana_rope* rope, void* ws,
                               size_t ws_bytes, void* hip_stream) {
  ProjGeometry g;
  int rc = make_proj_geometry(B, H, N, C, D, dtype, &g);
  if (rc != SANA_OK) return rc;
  if (g.BH == 0 || N == 0) return SANA_OK;
  if (check_tensor(x) || check_tensor(w_k) || check_tensor(w_v)) return SANA_ERR_INVALID;
  if (!kv_state || !ksum_state || !aligned(kv_state, 4) || !aligned(ksum_state, 4)) return SANA_ERR_INVALID;
  const size_t x_bytes = (size_t)B * N * C * 2, w_bytes = (size_t)H * la::kD * C * 2;
  const size_t kv_bytes = (size_t)g.BH * 1024 * sizeof(float), ks_bytes = (size_t)g.BH * 32 * sizeof(float);
  const void* ins[3] = {x, w_k, w_v};
  const size_t in_bytes[3] = {x_bytes, w_bytes, w_bytes};
  for (int i = 0; i < 3; ++i)
    if (overlaps(kv_state, kv_bytes, ins[i], in_bytes[i]) || overlaps(ksum_state, ks_bytes, ins[i], in_bytes[i]))
      return SANA_ERR_INVALID;
  if (overlaps(kv_state, kv_bytes, ksum_state, ks_bytes)) return SANA_ERR_INVALID;
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  if (!ws || ws_bytes < g.total_bytes) return SANA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SANA_ERR_INVALID;
  if ((rc = check_workspace_overlaps(ws, g.total_bytes,
                                     {{x, x_bytes}, {w_k, w_bytes}, {w_v, w_bytes}, {kv_state, kv_bytes},
                                      {ksum_state, ks_bytes}},
                                     rope)) != SANA_OK)
    return rc;

  la::ProjArgs p;
  p.x = static_cast<const char*>(x);
  p.wk = static_cast<const char*>(w_k);
  p.wv = static_cast<const char*>(w_v);
  p.N = N;
  p.C = C;
  p.H = H;
  p.Hp = (int)ceil_div(H, 4);
  p.R = g.R;
  p.T = g.T;
  p.M = (int64_t)B * g.R;
  p.G = (uint32_t)g.G;
  la::StateArgs a;
  a.partials = static_cast<float*>(ws);
  a.states = reinterpret_cast<float*>(static_cast<char*>(ws) + g.state_off);
  a.kv_in = kv_state;
  a.ksum_in = ksum_state;
  a.kv_out = kv_state;
  a.ksum_out = ksum_state;
  a.N = N;
  a.L = N;
  a.Ls = g.T * la::kProjTokens;
  a.C = 1;
  a.Pc = (int)g.R;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const RopeArg ra = rope_arg(rope, N);
  with_rope(ra.kind, [&](auto R) {
    constexpr int RO = decltype(R)::value;
    la::project_state_bf16<RO><<<dim3(la::proj_grid(p.G)), dim3(la::kProjThreads), 0, st>>>(p, ra.r, a);
  });
  if (g.R > 1) launch_finalize(a, g.BH, st);
  return launch_status();
}

int sana_linattn_project_apply(const void* x, const void* w_q, void* o, const sana_layout* out,
                               const float* kv_state, const float* ksum_state, int B, int H, int64_t N, int C, int D,
                               int dtype, float eps, const sana_rope* rope, void* hip_stream) {
  ProjGeometry pg;
  int rc = make_proj_geometry(B, H, N, C, D, dtype, &pg);
  if (rc != SANA_OK) return rc;
  if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID;
  if (pg.BH == 0 || N == 0) return SANA_OK;
  if (check_tensor(x) || check_tensor(w_q) || check_tensor(o)) return SANA_ERR_INVALID;
  if (!kv_state || !ksum_state || !aligned(kv_state, 4) || !aligned(ksum_state, 4)) return SANA_ERR_INVALID;
  View vout;
  if ((rc = make_view(out, B, H, N, D, 2, true, &vout)) != SANA_OK) return rc;
  const size_t x_bytes = (size_t)B * N * C * 2, w_bytes = (size_t)H * la::kD * C * 2;
  const size_t kv_bytes = (size_t)pg.BH * 1024 * sizeof(float), ks_bytes = (size_t)pg.BH * 32 * sizeof(float);
  const void* ins[4] = {x, w_q, kv_state, ksum_state};
  const size_t in_bytes[4] = {x_bytes, w_bytes, kv_bytes, ks_bytes};
  for (int i = 0; i < 4; ++i)
    if (overlaps(o, vout.span, ins[i], in_bytes[i])) return SANA_ERR_INVALID;
  if ((rc = check_rope(rope, N)) != SANA_OK) return rc;
  const int64_t nblk = ceil_div(N, la::kProjTokens);
  const int64_t groups = (int64_t)B * nblk * ceil_div(H, 8);
  if (groups > kMaxGroups) return SANA_ERR_INVALID;

  la::ProjApplyArgs p;
  p.x = static_cast<const char*>(x);
  p.wq = static_cast<const char*>(w_q);
  p.o = static_cast<char*>(o);
  p.lo = vout.lay;
  p.kv = kv_state;
  p.ks = ksum_state;
  p.N = N;
  p.C = C;
  p.H = H;
  p.Hq = (int)ceil_div(H, 8);
  p.R = nblk;
  p.M = (int64_t)B * nblk;
  p.G = (uint32_t)groups;
  p.eps = eps;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const RopeArg ra = rope_arg(rope, N);
  with_rope(ra.kind, [&](auto R) {
    constexpr int RO = decltype(R)::value;
    la::project_apply_bf16<RO><<<dim3(la::proj_grid(p.G)), dim3(la::kProjThreads), 0, st>>>(p, ra.r);
  });
  return launch_status();
}

const char* sana_linattn_source_hash(void) { return SANA_SOURCE_HASH; }

const char* sana_linattn_status_string(int status) {
  switch (status) {
    case SANA_OK: return "SANA_OK";
    case SANA_ERR_INVALID: return "SANA_ERR_INVALID: invalid argument";
    case SANA_ERR_UNSUPPORTED: return "SANA_ERR_UNSUPPORTED: unsupported head width (only D = 32)";
    case SANA_ERR_WORKSPACE: return "SANA_ERR_WORKSPACE: workspace missing or too small";
    case SANA_ERR_HIP: return "SANA_ERR_HIP: a HIP launch failed";
    default: return "unknown sana_status";
  }
}

}  // extern "C"
