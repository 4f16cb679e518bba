// HIP kernels (gfx950 / CDNA4) of SANA's ReLU linear attention.
//
// The method (phi = ReLU):
//   state pass   S = sum_j phi~(K_j)^T V_j, z = sum_j phi(K_j) per (batch, head)
//   apply pass   O_i = phi~(Q_i).S / (phi(Q_i).z + eps)
// "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion
// Transformers" (research note), Model architecture item 2) Linear DiT: the
// two shared sums are computed once and reused by every query.  "SANA-Video"
// paper notes 2.2: RoPE (phi~) is applied after the ReLU and only in the
// numerator; 2.3: the carried state is the running sum of S and z.
//
// Data layout: Q, K, V, O are [BH][N][32] views (see Layout: token n of head
// bh at a strided element offset) with the 32 features contiguous (64-byte
// rows in bf16).  Partial states are [BH][C][P][33][32] fp32: rows 0..31 hold
// S[d][e], row 32 holds z[d].  States are kv [BH][32][32] + ksum [BH][32].
//
// bf16 kernels put both 32-wide contractions on v_mfma_f32_16x16x32_bf16:
//   A (16x32) lane l holds row (l % 16), k-slice group (l / 16), 8 values;
//   B (32x16) lane l holds column (l % 16), k-slice group (l / 16), 8 values;
//   D (16x16) lane l holds column (l % 16), rows 4*(l / 16) + i, i = 0..3.
// The contraction pairs A slot (group, s) with B slot (group, s), so any
// assignment of physical indices to (group, slot) works as long as A and B use
// the same one; the kernels choose assignments that make every global load
// and store a contiguous 16-byte (apply) or 4-byte (state) lane access.
//
// Precision: bf16 x bf16 products are exact in fp32 and MFMA accumulates in
// fp32.  fp32 operands (the state in the apply pass, rotated features under
// RoPE) are split into three bf16 parts, x = hi + mid + lo, which is exact for
// any normal fp32 value (3 x 8 significant bits), and contracted with one MFMA
// per product term kept: with one exact bf16 operand that is 3 terms; with two
// split operands the 6 terms of weight >= 2^-16 (hh, hm, mh, hl, lh, mm).
//
// Sequence layout: each head's N tokens form C chunks of L tokens (the last may
// be shorter); a call without chunks has C = 1, L = N.  Each chunk is reduced
// by Pc workgroups ("splits").
//
// Reduction of the split-N partials: every state workgroup writes its partial
// (or, when a head has a single chunk and split, the finished state); a
// separate finalize kernel then walks each head's C x Pc partials in order
// (deterministic), adding them to the carried state, and stores the running
// sum at the end of every chunk: chunk c's state is S_in plus everything up
// to and including chunk c.  The kernel boundary makes the partials visible
// across all XCDs; an in-kernel hand-off would need an L2 write-back per
// publishing wave, which costs far more at this grid size.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kD = 32;               // head width (features per token)
constexpr int kStateElems = 33 * 32; // S (32x32) + z (32) per partial / state
constexpr int kThreads = 256;        // 4 wave64 per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));

// Geometry of the state pass and where its results go.
struct StateArgs {
  float* partials;                 // [BH][C][Pc][33][32] scratch (when C * Pc > 1)
  float* states;                   // [BH][C][33][32]: state of every chunk, read by the apply pass
  const float* kv_in;              // carried state [BH][32][32] or null (zero)
  const float* ksum_in;            // [BH][32] or null
  float* kv_out;                   // commit of the last chunk's state [BH][32][32] or null; may equal kv_in
  float* ksum_out;                 // [BH][32] or null; may equal ksum_in
  int64_t N;                       // tokens per head
  int64_t L;                       // tokens per chunk
  int64_t Ls;                      // tokens per split
  int C;                           // chunks per head
  int Pc;                          // splits per chunk
};

// Where the apply pass finds the state of (head bh, chunk c): S at
// s_base + (bh * C + c) * s_stride (32 x 32), z at z_base + (bh * C + c) * z_stride.
struct StateView {
  const float* s_base;
  const float* z_base;
  int64_t s_stride;
  int64_t z_stride;
};

// Where the tokens of a [B][H][N][32] tensor live: token n of head
// bh = b * H + h starts at element b * batch + h * head + n * token, and its
// 32 features are contiguous.  Contiguous [B][H][N][D] is
// {H*N*32, N*32, 32}; [B][N][H][D] is {N*H*32, 32, H*32}; the q, k or v part
// of a packed [B][N][3][H][D] projection output is {N*3*H*32, 32, 3*H*32}.
struct Layout {
  int64_t batch;
  int64_t head;
  int64_t token;
  int64_t H;

  // B*H < 2^24, so the head index splits with a 32-bit division; when the
  // batch stride continues the head stride (contiguous heads) none is needed.
  __device__ __forceinline__ int64_t base(int64_t bh) const {
    if (batch == H * head) return bh * head;
    const uint32_t b = (uint32_t)bh / (uint32_t)H;
    return (int64_t)b * batch + (int64_t)((uint32_t)bh - b * (uint32_t)H) * head;
  }
};

// ---------------------------------------------------------------------------
// RoPE angles
// ---------------------------------------------------------------------------
//
// Pair p of a token at position pos turns by an angle given in one of two
// forms (the kernels' ROPE template argument):
//   kRopeTable  cos/sin rows [pos][16] in device memory;
//   kRopeAxes   SANA-Video's 3D RoPE ("SANA-Video" paper notes, section 3
//               Stage 2): the latent point of pos = (t * Hl + h) * Wl + w,
//               pairs 0 .. pt-1 turn with t, the next ph with h, the rest with
//               w, by angles that depend on that one coordinate; so cos/sin are
//               per-axis tables [T][pt], [Hl][ph], [Wl][16-pt-ph] back to back
//               (a few KB; pt and ph even), which each workgroup stages in
//               LDS.
// Either way the angle values are the same floats, so the two forms give the
// same results bit for bit.
enum { kRopeNone = 0, kRopeTable = 1, kRopeAxes = 2 };
constexpr int kMaxAxisTab = 1024;  // floats per axis-form table (cos or sin)

struct Rope {
  const float* cos;
  const float* sin;
  int64_t pos0;      // position of token 0
  int64_t pos_last;  // last position in the call; axis lookups clamp to it
  int Hl, Wl;        // axis form: latent height and width
  int pt, ph;        // axis form: pairs turning with t and with h
  int base_h, base_w;  // axis form: offsets of the h and w tables
  int n_tab;         // axis form: floats per table
  double inv_w, inv_hw;  // axis form: 1 / Wl and 1 / (Hl * Wl)
};

// Axis form: the workgroup copies the tables to LDS in duos.  Entries 2d and
// 2d + 1 (with even pair counts per axis, two pairs of one axis at one
// coordinate) go to floats 4d .. 4d+3 as cos 2d, cos 2d+1, sin 2d, sin 2d+1,
// so one 16-byte read gives a duo's cosines and sines each in a register pair.
// The caller synchronises before the first lookup.
template <int ROPE>
__device__ __forceinline__ void rope_stage(const Rope& r, float* lds, int tid, int nthreads) {
  if constexpr (ROPE == kRopeAxes) {
    for (int d = tid; d < r.n_tab / 2; d += nthreads)
      *reinterpret_cast<f32x4_t*>(lds + 4 * d) =
          f32x4_t{r.cos[2 * d], r.cos[2 * d + 1], r.sin[2 * d], r.sin[2 * d + 1]};
  }
}

// cos/sin of staged entry e
__device__ __forceinline__ void axis_cs(const float* lds, int e, float& c, float& sn) {
  const float* d = lds + 4 * (e >> 1) + (e & 1);
  c = d[0];
  sn = d[2];
}

// cos e, cos e+1, sin e, sin e+1 of the duo that starts at staged entry e (even)
__device__ __forceinline__ f32x4_t axis_duo(const float* lds, int e) {
  return *reinterpret_cast<const f32x4_t*>(lds + 2 * e);
}

// Latent coordinates of position pos (clamped to the call's last position),
// by double-precision reciprocals: floor((n + 1/2) / d) is exact for n < 2^31
// and d < 2^20, as the fraction stays 1/(2d) away from an integer.  Positions
// stay below 2^32 (the last is below 2^31, a tile reaches a few past it), so
// the clamp is 32-bit.
__device__ __forceinline__ void rope_coords(const Rope& r, int64_t pos, int& t, int& h, int& w) {
  const unsigned last = (unsigned)r.pos_last;
  const unsigned n = (unsigned)pos < last ? (unsigned)pos : last;
  t = (int)__builtin_fma((double)n, r.inv_hw, 0.5 * r.inv_hw);
  const int rem = (int)n - t * (r.Hl * r.Wl);
  h = (int)__builtin_fma((double)rem, r.inv_w, 0.5 * r.inv_w);
  w = rem - (int)__umul24(h, r.Wl);  // h Wl <= rem < Hl Wl < 2^20
}

// Where pair p's entry sits, as offset + t * wt + h * wh + w * ww: one of the
// three weights is the pair count of p's axis, the others 0.
struct AxisPair {
  int off, wt, wh, ww;
};

__device__ __forceinline__ AxisPair axis_pair(const Rope& r, int p) {
  const int pw = 16 - r.pt - r.ph;
  if (p < r.pt) return AxisPair{p, r.pt, 0, 0};
  if (p < r.pt + r.ph) return AxisPair{r.base_h + p - r.pt, 0, r.ph, 0};
  return AxisPair{r.base_w + p - r.pt - r.ph, 0, 0, pw};
}

// 24-bit products (full rate): the one non-zero weight's coordinate times it
// stays below the table size (at most kMaxAxisTab), and a zero weight gives 0
// whatever the coordinate's high bits.
__device__ __forceinline__ int axis_entry(const AxisPair& a, int t, int h, int w) {
  return (int)(__umul24(t, a.wt) + __umul24(h, a.wh) + __umul24(w, a.ww)) + a.off;
}

// A lane's pairs 4g .. 4g+3 as two duos (4g, 4g+1) and (4g+2, 4g+3): the axis
// form has even pair counts per axis, so each duo sits in one axis, at
// consecutive entries.
struct AxisLane {
  AxisPair duo[2];
};

__device__ __forceinline__ AxisLane axis_lane(const Rope& r, int g) {
  return AxisLane{{axis_pair(r, 4 * g), axis_pair(r, 4 * g + 2)}};
}

// cos/sin of pairs 4g .. 4g+3 of position pos from the staged tables: one
// 16-byte LDS read (cos, sin of both pairs) per duo.
__device__ __forceinline__ void rope_axis_row4(const Rope& r, const float* lds, const AxisLane& al,
                                               int64_t pos, f32x4_t& c, f32x4_t& sn) {
  int t, h, w;
  rope_coords(r, pos, t, h, w);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const f32x4_t e = axis_duo(lds, axis_entry(al.duo[d], t, h, w));
    c[2 * d] = e[0];
    c[2 * d + 1] = e[1];
    sn[2 * d] = e[2];
    sn[2 * d + 1] = e[3];
  }
}

// cos/sin of pair p of position pos, in either form (`lds`: the staged tables).
template <int ROPE>
__device__ __forceinline__ void rope_pair(const Rope& r, const float* lds, int64_t pos, int p, float& c, float& sn) {
  if constexpr (ROPE == kRopeAxes) {
    int t, h, w;
    rope_coords(r, pos, t, h, w);
    axis_cs(lds, axis_entry(axis_pair(r, p), t, h, w), c, sn);
  } else {
    c = r.cos[pos * 16 + p];
    sn = r.sin[pos * 16 + p];
  }
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

// ReLU of two packed bf16: a bf16 with the sign bit set is a negative int16,
// so a signed 16-bit max against 0 clears it (and maps -0 to +0).
__device__ __forceinline__ unsigned relu_bf16x2(unsigned x) {
  const s16x2_t zero = {0, 0};
  return __builtin_bit_cast(unsigned, __builtin_elementwise_max(__builtin_bit_cast(s16x2_t, x), zero));
}

__device__ __forceinline__ float bf16lo_to_f32(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi_to_f32(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

// One RoPE pair rotation, (a, b) -> (a c - b s, a s + b c), with its fused
// multiply-adds written out: left to the compiler, the contraction may fuse
// either product of a c - b s depending on the surrounding code, and two
// kernels (or two table forms) inlining the same source could round apart.
__device__ __forceinline__ float rot_lo(float a, float b, float c, float s) { return __builtin_fmaf(a, c, -(b * s)); }
__device__ __forceinline__ float rot_hi(float a, float b, float c, float s) { return __builtin_fmaf(a, s, b * c); }

// A constant the compiler cannot see through, held in an SGPR.  The packed
// bf16 operand below must reach the instruction as these exact bits: folded
// into an inline constant, (-1.0, 0) is encoded as the fp32 inline -1.0, which
// the hardware reads as (0, -1.0).
__device__ __forceinline__ unsigned sgpr_constant(unsigned x) {
  asm("" : "+s"(x));
  return x;
}

// x minus the bf16 in the low (high) half of `packed`, as one bf16 dot product
// (v_dot2c_f32_bf16) against (-1, 0) (against (0, -1)): both products are
// exact and, for the bf16 rounding of x, so is the difference (x - bf16(x)
// has at most 16 significant bits), so the instruction's one rounding changes
// nothing.  It replaces an unpack and a subtraction.  The other half enters
// as a product with 0, which is NaN only if that half is infinite.
__device__ __forceinline__ float minus_lo_bf16(unsigned packed, float x) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed),
                                         __builtin_bit_cast(bf16x2_t, sgpr_constant(0x0000bf80u)), x, false);
}
__device__ __forceinline__ float minus_hi_bf16(unsigned packed, float x) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed),
                                         __builtin_bit_cast(bf16x2_t, sgpr_constant(0xbf800000u)), x, false);
}

// x = hi + mid + lo with hi = bf16(x), mid = bf16(x - hi), lo = bf16(x - hi - mid);
// each residual is exact in fp32 (x - bf16(x) has at most 16 significant
// bits).  Called for a pair (a, b), each part comes back as one dword of two
// packed bf16.
__device__ __forceinline__ void split3_bf16x2(float a, float b, unsigned& hi, unsigned& mid, unsigned& lo) {
  hi = pack_bf16x2(a, b);
  const float ra = minus_lo_bf16(hi, a), rb = minus_hi_bf16(hi, b);
  mid = pack_bf16x2(ra, rb);
  lo = pack_bf16x2(minus_lo_bf16(mid, ra), minus_hi_bf16(mid, rb));
}

__device__ __forceinline__ unsigned lo_halves(unsigned a, unsigned b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ unsigned hi_halves(unsigned a, unsigned b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(unsigned a, unsigned b, unsigned c, unsigned d) {
  const u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}

// even (low) halves of 8 dwords as 8 bf16, and odd (high) halves
__device__ __forceinline__ bf16x8_t even8(const unsigned (&x)[8]) {
  return as_bf16x8(lo_halves(x[0], x[1]), lo_halves(x[2], x[3]), lo_halves(x[4], x[5]), lo_halves(x[6], x[7]));
}
__device__ __forceinline__ bf16x8_t odd8(const unsigned (&x)[8]) {
  return as_bf16x8(hi_halves(x[0], x[1]), hi_halves(x[2], x[3]), hi_halves(x[4], x[5]), hi_halves(x[6], x[7]));
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Buffer access
// ---------------------------------------------------------------------------
//
// The bf16 kernels address memory through buffer resources built in SGPRs, one
// per 64-token chunk, whose size is the number of bytes left before the end of
// the token range: the hardware range check then reads rows past the end as 0
// and drops stores past it, so the loops need no per-lane predicates and no
// 64-bit address arithmetic (lane offsets are 32-bit, tile offsets immediate).
// The range check covers the per-lane offset plus the immediate, which is all
// the kernels use.

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer
constexpr int kNonTemporal = 2;         // cache policy of data streamed once

// `bytes` from `base` are in range.  The callers touch at most a few KB past
// `base`, so clamping a larger size to what the descriptor holds cuts nothing.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t nr = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nr, kRsrcWord3);
}

// Descriptor for rows t0 .. n_end-1 of a tensor whose rows are `row` bytes
// apart (64 of them in use): rows at or past n_end fall outside.
__device__ __forceinline__ rsrc_t rows_rsrc(const char* head_base, int64_t t0, int64_t n_end, int64_t row) {
  return make_rsrc(head_base + t0 * row, (n_end - t0 - 1) * row + 64);
}

__device__ __forceinline__ u32x4_t load16_nt(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}

// Streamed rows are loaded non-temporal, unless another wave of the workgroup
// reads the other half of the same 128-byte lines (two heads per workgroup):
// then the line must stay in L2 until that wave's load arrives.
template <int HEADS>
__device__ __forceinline__ u32x4_t load16_stream(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, HEADS == 1 ? kNonTemporal : 0));
}

__device__ __forceinline__ f32x4_t load16(rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float load4(rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void store16_nt(rsrc_t r, int off, u32x4_t x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, off, 0, kNonTemporal);
}

// ---------------------------------------------------------------------------
// Writing a workgroup's partial state, and the finalize kernel
// ---------------------------------------------------------------------------

// Element idx (33 x 32 layout) of the carried state, 0 when there is none.
__device__ __forceinline__ float carried_state(const float* kv_in, const float* ksum_in, int64_t bh, int idx) {
  if (idx < 1024) return kv_in ? kv_in[bh * 1024 + idx] : 0.f;
  return ksum_in ? ksum_in[bh * 32 + (idx - 1024)] : 0.f;
}

__device__ __forceinline__ float carried(const StateArgs& a, int64_t bh, int idx) {
  return carried_state(a.kv_in, a.ksum_in, bh, idx);
}

// Stores element idx of the last chunk's state as the committed state.
__device__ __forceinline__ void commit(const StateArgs& a, int64_t bh, int idx, float x) {
  if (idx < 1024)
    a.kv_out[bh * 1024 + idx] = x;
  else
    a.ksum_out[bh * 32 + (idx - 1024)] = x;
}

// `mine` (LDS, 33x32 floats) holds this workgroup's sum for head bh, chunk c,
// split s.  With a single chunk and split it is already the head's sum: it
// goes, with the carried state added, straight to the state (and the
// commit); otherwise it is stored as a partial.
__device__ __forceinline__ void write_partial(const float* mine, int64_t bh, int c, int s, const StateArgs& a,
                                              int tid = threadIdx.x) {
  if (a.C * a.Pc == 1) {
    for (int idx = tid; idx < kStateElems; idx += kThreads) {
      const float x = carried(a, bh, idx) + mine[idx];
      a.states[bh * kStateElems + idx] = x;
      if (a.kv_out) commit(a, bh, idx, x);
    }
  } else {
    float* out = a.partials + (((int64_t)bh * a.C + c) * a.Pc + s) * kStateElems;
    for (int idx = tid; idx < kStateElems; idx += kThreads) out[idx] = mine[idx];
  }
}

// One thread per state element of every head.  It walks the head's C x Pc
// partials in order, BATCH loads in flight at a time, adding each to the
// carried state, and stores the running sum at the end of every chunk; the
// last one is also committed.  kv_out may alias kv_in: each element is read
// and written by the same thread.
//
// The loads of a batch go out unconditionally, those past the head's last
// partial reading that partial again (unused): a predicated load per partial
// leaves the compiler unable to keep them in flight together.  The host takes
// BATCH = 16 for up to 16 partials per head and 64 above: the fused
// projections leave one partial per 256-token range, 64-73 per head on the
// large layers, and a wave then has 64 x 256 B in flight instead of walking
// them in four or five round trips.
template <int BATCH>
__global__ __launch_bounds__(kThreads) void state_finalize(StateArgs a, int64_t n_elems) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_elems) return;
  const int64_t bh = i / kStateElems;
  const int idx = (int)(i % kStateElems);
  const int total = a.C * a.Pc;
  const float* src = a.partials + bh * total * kStateElems + idx;
  float* dst = a.states + bh * a.C * kStateElems + idx;
  float acc = carried(a, bh, idx);
  int c = 0, s = 0;  // chunk and split of the next partial
  for (int q0 = 0; q0 < total; q0 += BATCH) {
    float v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) v[u] = src[(int64_t)min(q0 + u, total - 1) * kStateElems];
    const int nb = total - q0;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (u < nb) {
        acc += v[u];
        if (++s == a.Pc) {
          dst[(int64_t)c * kStateElems] = acc;
          s = 0;
          ++c;
        }
      }
    }
  }
  if (a.kv_out) commit(a, bh, idx, acc);
}

// Token range [n_begin, n_end) of state workgroup (bh, c, s) = blockIdx.x,
// numbered head-major, or (units > 0) head-minor over `units` heads or head
// pairs, so that workgroups launched together read the same tokens.
__device__ __forceinline__ void state_item(const StateArgs& a, int64_t& bh, int& c, int& s, int64_t& n_begin,
                                           int64_t& n_end, int64_t units = 0) {
  const int per_head = a.C * a.Pc;
  int r;
  if (units > 0) {
    bh = blockIdx.x % units;
    r = (int)(blockIdx.x / units);
  } else {
    bh = blockIdx.x / per_head;
    r = blockIdx.x % per_head;
  }
  c = r / a.Pc;
  s = r % a.Pc;
  const int64_t c_begin = (int64_t)c * a.L;
  const int64_t c_end = (c_begin + a.L < a.N) ? c_begin + a.L : a.N;
  n_begin = c_begin + (int64_t)s * a.Ls;
  n_end = (n_begin + a.Ls < c_end) ? n_begin + a.Ls : c_end;
}

// The same items dealt XCD by XCD: workgroup b runs on XCD b % 8 (MI355X), and
// heads x, x + 8, x + 16, ... take the slots b / 8 of XCD x, all of a head's
// items on one XCD.  Slots past the last head are left without a head
// (bh >= BH).  For the apply that sums the partials itself (apply_fold_bf16),
// whose workgroups of a head sit on the same XCD.
constexpr int kXcdCount = 8;

__device__ __forceinline__ void state_item_xcd(const StateArgs& a, int64_t& bh, int& c, int& s, int64_t& n_begin,
                                               int64_t& n_end) {
  const int per_head = a.C * a.Pc;
  const int slot = blockIdx.x / kXcdCount;
  bh = blockIdx.x % kXcdCount + (int64_t)kXcdCount * (slot / per_head);
  const int r = slot % per_head;
  c = r / a.Pc;
  s = r % a.Pc;
  const int64_t c_begin = (int64_t)c * a.L;
  const int64_t c_end = (c_begin + a.L < a.N) ? c_begin + a.L : a.N;
  n_begin = c_begin + (int64_t)s * a.Ls;
  n_end = (n_begin + a.Ls < c_end) ? n_begin + a.Ls : c_end;
}

// ---------------------------------------------------------------------------
// bf16 state pass: split-N partial S and z with MFMA
// ---------------------------------------------------------------------------
//
// One workgroup reduces tokens [s*Ls, min(N, (s+1)*Ls)) of one (batch, head);
// its four waves take 32-token tiles, two at a time.  With HEADS = 2 it has
// eight waves and takes heads 2u and 2u + 1 of the same tokens, four waves
// each, exactly as two one-head workgroups would: when adjacent heads share
// each 128-byte line (a [B][N][H][D] or packed QKV layout), both halves of every
// line are then read by one CU at the same time.  Such layouts interleave the
// heads of a token, so those workgroups are numbered head-minor: the ones
// launched together take every head of the same tokens, and a DRAM page
// holding one token's heads is read by all of them at about the same time.
//
// The contraction runs over tokens, but rows in memory are token-major.  Each
// lane therefore loads whole-row pieces -- lane l (n = l % 16, g = l / 16)
// reads the 16 bytes holding features 8g .. 8g+7 of token t0 + 16tb + n, so a
// wave reads 16 rows (1 KB contiguous) per load -- and the rows are turned
// around on the matrix core: with the tile as A (row = token, k = feature) and
// a 0/1 selection matrix E_fh as B (E_fh[k][c] = [k == 16fh + c]), the MFMA
// returns D[token][c] = X[token][16fh + c] in the D layout, i.e. lane (n, g)
// holds feature 16fh + n of tokens t0 + 16tb + 4g + i, i = 0..3.  The values
// are bf16 times 1.0, so the turn-around is exact.  Packed back to bf16,
// those are exactly the operands of the token contraction:
//   A_fh (rows = key features 16fh + n, k-slots = the lane group's 8 tokens)
//   B_fh (columns = value features 16fh + n, same token slots)
// and S[16fh + 4g + i][16fh' + n] accumulates in MFMA (fh, fh').  Two more
// MFMAs against a B of ones give z.
//
// Under RoPE the rotation acts on pairs (2p, 2p+1) of a token.  It is applied
// after the turn-around, where lane (n, g) holds feature f = 16fh + n of
// tokens t0 + 16tb + 4g + i: a second selection MFMA hands the lane the pair
// partner f ^ 1 with the rotation's sign, cos/sin of pair f / 2 are gathered
// per token, and the rotated fp32 values are split into three bf16 parts that
// are contracted against V one by one.  z always comes from the un-rotated
// phi(K).

// E_fh as the B operand of lane (n, g): slot s is 1.0 where 8g + s == 16fh + n
__device__ __forceinline__ bf16x8_t select_operand(int g, int n, int fh) {
  unsigned d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int k = 8 * g + 2 * p;
    d[p] = (k == 16 * fh + n ? 0x3f80u : 0u) | (k + 1 == 16 * fh + n ? 0x3f800000u : 0u);
  }
  return as_bf16x8(d[0], d[1], d[2], d[3]);
}

// The pair partner's selection: slot s is where 8g + s == (16fh + n) ^ 1, with
// value -1.0 for even n and +1.0 for odd n, so the turn-around returns
// -x[f + 1] (f even) or +x[f - 1] (f odd) and the rotated value is
// x[f] cos + partner sin (pair p: (x0 c - x1 s, x0 s + x1 c)).
__device__ __forceinline__ bf16x8_t partner_operand(int g, int n, int fh) {
  const int f = (16 * fh + n) ^ 1;
  const unsigned one = (n & 1) ? 0x3f80u : 0xbf80u;
  unsigned d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int k = 8 * g + 2 * p;
    d[p] = (k == f ? one : 0u) | (k + 1 == f ? one << 16 : 0u);
  }
  return as_bf16x8(d[0], d[1], d[2], d[3]);
}

// Turn-around of one 16-token half (exact: bf16 values times 1.0)
__device__ __forceinline__ f32x4_t turn(bf16x8_t x, bf16x8_t sel) {
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  return mfma16(x, sel, zero4);
}

// Turned-around halves tb = 0, 1 of one feature half -> bf16 operand
__device__ __forceinline__ bf16x8_t pack_turned(f32x4_t t0, f32x4_t t1) {
  return as_bf16x8(pack_bf16x2(t0[0], t0[1]), pack_bf16x2(t0[2], t0[3]), pack_bf16x2(t1[0], t1[1]),
                   pack_bf16x2(t1[2], t1[3]));
}

__device__ __forceinline__ u32x4_t relu_bf16x8(u32x4_t x) {
  x[0] = relu_bf16x2(x[0]);
  x[1] = relu_bf16x2(x[1]);
  x[2] = relu_bf16x2(x[2]);
  x[3] = relu_bf16x2(x[3]);
  return x;
}

// pack_turned's words, passed through an empty asm: where a ReLU of the packed
// bf16 follows, the compiler would otherwise split each two-float conversion
// into two one-float conversions and a v_perm (three instructions for one).
__device__ __forceinline__ u32x4_t pack_turned_words(f32x4_t t0, f32x4_t t1) {
  unsigned w0 = pack_bf16x2(t0[0], t0[1]), w1 = pack_bf16x2(t0[2], t0[3]);
  unsigned w2 = pack_bf16x2(t1[0], t1[1]), w3 = pack_bf16x2(t1[2], t1[3]);
  asm("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
  return u32x4_t{w0, w1, w2, w3};
}

// phi of a freshly computed tile: pack_turned, then the ReLU of the packed bf16
__device__ __forceinline__ u32x4_t pack_turned_relu(f32x4_t t0, f32x4_t t1) {
  return relu_bf16x8(pack_turned_words(t0, t1));
}

// cos and sin that lane (n, g) needs for a 32-token tile at t0: element
// [fh][tb][i] belongs to pair 8fh + n / 2 of token t0 + 16tb + 4g + i.  They
// are loaded like K (16-byte row pieces: lane (n, g) gets pairs 4g .. 4g+3 of
// token t0 + 16tb + n; rows at or past n_end read 0, as does their phi(K)) and
// turned around through a wave-private LDS tile, [cos | sin][32 rows][kAngRow]
// floats: with rows of 18 floats the 16 lanes of each group g read 8
// consecutive banks of their own.
constexpr int kAngRow = 18;
constexpr int kAngTile = 2 * 32 * kAngRow;  // floats per wave

struct TileAngles {
  f32x4_t c[2][2], s[2][2];
};

struct TileAnglesRows {
  f32x4_t c[2], s[2];
};

__device__ __forceinline__ void load_angle_rows(const float* cos_t, const float* sin_t, int64_t pos0, int64_t t0,
                                                int64_t n_end, int tab_off, TileAnglesRows& rows) {
  const rsrc_t rc = make_rsrc(cos_t + (pos0 + t0) * 16, (n_end - t0) * 64);
  const rsrc_t rs = make_rsrc(sin_t + (pos0 + t0) * 16, (n_end - t0) * 64);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    rows.c[tb] = load16(rc, tab_off + tb * 1024);
    rows.s[tb] = load16(rs, tab_off + tb * 1024);
  }
}

// Every lane of the wave writes and then reads the tile: the wavefront-scope
// fences keep the compiler from moving LDS accesses across them (a wave's LDS
// accesses are performed in order, so no wait is needed).
__device__ __forceinline__ void turn_angles(const TileAnglesRows& rows, float* lds, int g, int n, TileAngles& ang) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    float* rc = lds + (16 * tb + n) * kAngRow + 4 * g;
    float* rs = rc + 32 * kAngRow;
    *reinterpret_cast<float2*>(rc) = float2{rows.c[tb][0], rows.c[tb][1]};
    *reinterpret_cast<float2*>(rc + 2) = float2{rows.c[tb][2], rows.c[tb][3]};
    *reinterpret_cast<float2*>(rs) = float2{rows.s[tb][0], rows.s[tb][1]};
    *reinterpret_cast<float2*>(rs + 2) = float2{rows.s[tb][2], rows.s[tb][3]};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* rc = lds + (16 * tb + 4 * g + i) * kAngRow + (n >> 1);
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        ang.c[fh][tb][i] = rc[8 * fh];
        ang.s[fh][tb][i] = rc[32 * kAngRow + 8 * fh];
      }
    }
}

// acc[fh][fh']: S blocks (key half fh, value half fh'); accz[fh]: z of key half fh
template <bool ROPE>
__device__ __forceinline__ void state_tile(const u32x4_t (&kx)[2], const u32x4_t (&vx)[2],
                                           const TileAnglesRows& rows, int g, int n, float* lds,
                                           const bf16x8_t (&sel)[2], const bf16x8_t (&selp)[2],
                                           f32x4_t (&acc)[2][2], f32x4_t (&accz)[2]) {
  const unsigned one2 = 0x3f803f80u;  // two bf16 1.0
  const bf16x8_t ones = as_bf16x8(one2, one2, one2, one2);
  bf16x8_t k_nat[2], v_nat[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    k_nat[tb] = __builtin_bit_cast(bf16x8_t, relu_bf16x8(kx[tb]));
    v_nat[tb] = __builtin_bit_cast(bf16x8_t, vx[tb]);
  }
  f32x4_t kt[2][2];  // [fh][tb]: phi(K) turned around, exact fp32
  bf16x8_t a[2], b[2];
#pragma unroll
  for (int fh = 0; fh < 2; ++fh) {
    kt[fh][0] = turn(k_nat[0], sel[fh]);
    kt[fh][1] = turn(k_nat[1], sel[fh]);
    a[fh] = pack_turned(kt[fh][0], kt[fh][1]);
    b[fh] = pack_turned(turn(v_nat[0], sel[fh]), turn(v_nat[1], sel[fh]));
  }
#pragma unroll
  for (int fh = 0; fh < 2; ++fh) accz[fh] = mfma16(a[fh], ones, accz[fh]);
  if constexpr (!ROPE) {
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
      acc[fh][0] = mfma16(a[fh], b[0], acc[fh][0]);
      acc[fh][1] = mfma16(a[fh], b[1], acc[fh][1]);
    }
  } else {
    TileAngles ang;
    turn_angles(rows, lds, g, n, ang);
    unsigned part[3][2][4];  // [bf16 part][fh][dword]: the slot order of a[fh]
#pragma unroll
    for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const f32x4_t xp = turn(k_nat[tb], selp[fh]);
        f32x4_t y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = kt[fh][tb][i] * ang.c[fh][tb][i] + xp[i] * ang.s[fh][tb][i];
        split3_bf16x2(y[0], y[1], part[0][fh][2 * tb], part[1][fh][2 * tb], part[2][fh][2 * tb]);
        split3_bf16x2(y[2], y[3], part[0][fh][2 * tb + 1], part[1][fh][2 * tb + 1], part[2][fh][2 * tb + 1]);
      }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        const bf16x8_t ar = as_bf16x8(part[k][fh][0], part[k][fh][1], part[k][fh][2], part[k][fh][3]);
        acc[fh][0] = mfma16(ar, b[0], acc[fh][0]);
        acc[fh][1] = mfma16(ar, b[1], acc[fh][1]);
      }
    }
  }
}

// One wave's share of a token range of one head: the 64-token chunks at t0,
// t0 + 256, ... below n_end (a workgroup's four waves start 64 tokens apart),
// accumulated into acc (S blocks, key half fh x value half fh') and accz (z).
// The next chunk's loads are issued before the current chunk is computed.
// `row`: bytes between tokens; `lds`: the wave's angle tile (RoPE only);
// `rtab`: the staged per-axis tables (axis form only).
template <int ROPE, int HEADS>
__device__ __forceinline__ void state_accumulate(const char* Kh, const char* Vh, int64_t row, int64_t t0,
                                                 int64_t n_end, const Rope& rp, const float* rtab, float* lds, int g,
                                                 int n, f32x4_t (&acc)[2][2], f32x4_t (&accz)[2]) {
  const AxisLane al = axis_lane(rp, g);  // axis form only
  // lane's 16-byte piece of a row: features 8g .. 8g+7 of token (tile row) n
  const int lane_off = n * (int)row + g * 16;
  const int tab_off = n * 64 + g * 16;  // the same piece of a cos/sin table row

  const bf16x8_t sel[2] = {select_operand(g, n, 0), select_operand(g, n, 1)};
  const bf16x8_t selp[2] = {partner_operand(g, n, 0), partner_operand(g, n, 1)};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    accz[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[i][0] = accz[i];
    acc[i][1] = accz[i];
  }

  // each wave takes 64-token chunks (two 32-token tiles of two 16-row halves)
  u32x4_t nk[4], nv[4];
  TileAnglesRows na[2];  // cos/sin rows of the two tiles (RoPE only)
  auto load_chunk = [&](int64_t c0) {
    const rsrc_t rk = rows_rsrc(Kh, c0, n_end, row);
    const rsrc_t rv = rows_rsrc(Vh, c0, n_end, row);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      nk[h] = load16_stream<HEADS>(rk, lane_off + h * 16 * (int)row);
      nv[h] = load16_stream<HEADS>(rv, lane_off + h * 16 * (int)row);
    }
    if constexpr (ROPE == kRopeTable) {
      load_angle_rows(rp.cos, rp.sin, rp.pos0, c0, n_end, tab_off, na[0]);
      load_angle_rows(rp.cos, rp.sin, rp.pos0, c0 + 32, n_end, tab_off, na[1]);
    }
    // the axis form's angles come from LDS when the tile is computed
  };
  if (t0 < n_end) load_chunk(t0);
  for (; t0 < n_end; t0 += 256) {
    const u32x4_t ka[2] = {nk[0], nk[1]}, va[2] = {nv[0], nv[1]};
    const u32x4_t kb[2] = {nk[2], nk[3]}, vb[2] = {nv[2], nv[3]};
    TileAnglesRows ra = na[0], rb = na[1];
    if (t0 + 256 < n_end) load_chunk(t0 + 256);
    if constexpr (ROPE == kRopeAxes) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 16 * tb + n, ra.c[tb], ra.s[tb]);
        rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 32 + 16 * tb + n, rb.c[tb], rb.s[tb]);
      }
    }
    state_tile<ROPE != 0>(ka, va, ra, g, n, lds, sel, selp, acc, accz);
    if (t0 + 32 < n_end) state_tile<ROPE != 0>(kb, vb, rb, g, n, lds, sel, selp, acc, accz);
  }
}

// A wave's accumulators into its 33 x 32 LDS tile.  D lane (n, g): rows
// 4g + i -> key feature 16fh + 4g + i, column n -> value feature 16fh' + n.
__device__ __forceinline__ void state_to_lds(const f32x4_t (&acc)[2][2], const f32x4_t (&accz)[2], float* rw, int g,
                                             int n) {
#pragma unroll
  for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * fh + 4 * g + i;
      rw[d * 32 + n] = acc[fh][0][i];
      rw[d * 32 + 16 + n] = acc[fh][1][i];
      if (n == 0) rw[1024 + d] = accz[fh][i];
    }
  }
}

// The four waves' tiles of r[0..3] summed into r[0], in a fixed order.
__device__ __forceinline__ void sum_wave_tiles(float (*r)[kStateElems], int tid) {
  for (int idx = tid; idx < kStateElems; idx += kThreads)
    r[0][idx] = (r[0][idx] + r[1][idx]) + (r[2][idx] + r[3][idx]);
}

// DENSE: consecutive tokens are adjacent 64-byte rows (token stride = 32
// elements), so every tile offset is an instruction immediate.
// XCD: items dealt by state_item_xcd (one head per workgroup only).
template <int ROPE, bool DENSE, int HEADS, bool XCD = false>
__global__ __launch_bounds__(kThreads* HEADS) void state_bf16(const u32x4_t* __restrict__ K,
                                                              const u32x4_t* __restrict__ V, Layout lkv, Rope rp,
                                                              StateArgs a, int64_t BH) {
  __shared__ float red[4 * HEADS][kStateElems];
  __shared__ float angles[ROPE ? 4 * HEADS : 1][ROPE ? kAngTile : 1];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads * HEADS);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  int64_t bh, n_begin, n_end;
  int c, s;
  if constexpr (XCD) {
    static_assert(HEADS == 1, "XCD-dealt items take one head per workgroup");
    state_item_xcd(a, bh, c, s, n_begin, n_end);
  } else {
    state_item(a, bh, c, s, n_begin, n_end, HEADS == 2 ? (BH + 1) / 2 : 0);
  }
  const int lane = threadIdx.x & 63;
  const int wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wg >> 2;  // which of the workgroup's heads
  const int w = wg & 3;      // wave within that head's four
  bh = bh * HEADS + half;
  const bool active = bh < BH;
  const int n = lane & 15;
  const int g = lane >> 4;

  const int64_t row = DENSE ? 64 : lkv.token * 2;  // bytes between tokens
  const char* Kh = reinterpret_cast<const char*>(K) + lkv.base(bh) * 2;
  const char* Vh = reinterpret_cast<const char*>(V) + lkv.base(bh) * 2;
  f32x4_t acc[2][2], accz[2];
  state_accumulate<ROPE, HEADS>(Kh, Vh, row, active ? n_begin + 64 * w : n_end, n_end, rp, rtab,
                                angles[ROPE ? wg : 0], g, n, acc, accz);
  state_to_lds(acc, accz, red[wg], g, n);
  __syncthreads();
  const int tid = threadIdx.x & (kThreads - 1);
  sum_wave_tiles(red + 4 * half, tid);
  __syncthreads();
  if (active) write_partial(red[4 * half], bh, c, s, a, tid);
}

// ---------------------------------------------------------------------------
// fp32 state pass (VALU): each thread owns S[d][e0..e0+3] (and z[d])
// ---------------------------------------------------------------------------
template <int ROPE>
__global__ __launch_bounds__(kThreads) void state_f32(const float* __restrict__ K, const float* __restrict__ V,
                                                      Layout lkv, Rope rp, StateArgs a) {
  __shared__ float sk[64][kD + 1];   // phi(K), un-rotated
  __shared__ float skr[64][kD + 1];  // phi~(K), rotated (RoPE only)
  __shared__ float sv[64][kD + 1];
  __shared__ float mine[kStateElems];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();

  int64_t bh, n_begin, n_end;
  int c, s;
  state_item(a, bh, c, s, n_begin, n_end);
  const int t = threadIdx.x;
  const int d = t >> 3;
  const int e0 = (t & 7) * 4;
  const float* Kh = K + lkv.base(bh);
  const float* Vh = V + lkv.base(bh);

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  for (int64_t t0 = n_begin; t0 < n_end; t0 += 64) {
    // 64 tokens x 16 pairs = 1024 pairs, 4 per thread
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pidx = t + kThreads * i;
      const int tok = pidx >> 4;
      const int p = pidx & 15;
      const int64_t gt = t0 + tok;
      float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
      if (gt < n_end) {
        k0 = fmaxf(Kh[gt * lkv.token + 2 * p], 0.f);
        k1 = fmaxf(Kh[gt * lkv.token + 2 * p + 1], 0.f);
        v0 = Vh[gt * lkv.token + 2 * p];
        v1 = Vh[gt * lkv.token + 2 * p + 1];
      }
      sk[tok][2 * p] = k0;
      sk[tok][2 * p + 1] = k1;
      sv[tok][2 * p] = v0;
      sv[tok][2 * p + 1] = v1;
      if constexpr (ROPE) {
        float c = 1.f, sn = 0.f;
        if (gt < n_end) rope_pair<ROPE>(rp, rtab, rp.pos0 + gt, p, c, sn);
        skr[tok][2 * p] = rot_lo(k0, k1, c, sn);
        skr[tok][2 * p + 1] = rot_hi(k0, k1, c, sn);
      }
    }
    __syncthreads();
    for (int j = 0; j < 64; ++j) {
      const float x = ROPE ? skr[j][d] : sk[j][d];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = fmaf(x, sv[j][e0 + c], acc[c]);
      zacc += sk[j][d];
    }
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) mine[d * 32 + e0 + c] = acc[c];
  if (e0 == 0) mine[1024 + d] = zacc;
  __syncthreads();
  write_partial(mine, bh, c, s, a);
}

// ---------------------------------------------------------------------------
// bf16 apply pass: O = phi~(Q).S / (phi(Q).z + eps) with MFMA
// ---------------------------------------------------------------------------
//
// Computed transposed, O^T (32 e x 16 tokens) = S^T (32 e x 32 d) . phi(Q)^T.
// Lane l (m = l % 16, g = l / 16) loads the 16 bytes holding features
// 8g .. 8g+7 of token t0 + m, so one load instruction of the wave reads 16
// whole rows (1 KB contiguous).  Slot s of group g is feature d = 8g + s.
// The 32 output features are two MFMAs of 16 rows; MFMA h row r maps to
// e = 8(r / 4) + 4h + (r % 4), so lane l ends with e = 8g .. 8g+7 of its token
// and stores them as one 16-byte write.  A third MFMA group whose rows all hold
// z gives the denominator of the lane's token in every accumulator.
//
// Work split: the B*H*N tokens, flattened head-major, are cut into equal
// contiguous ranges, one per workgroup; a range that crosses a head boundary
// is processed head segment by head segment.  Each wave takes 64-token chunks
// (four 16-token tiles, four loads in flight) of the current segment.  With
// HEADS = 2 the workgroup's eight waves take the same tokens of heads 2u and
// 2u + 1, four waves each, and workgroups are numbered head-minor: blockIdx.x
// = blk * units + u takes tokens [blk * La, (blk + 1) * La) of pair u (see the
// state pass).

struct ApplyOperands {
  bf16x8_t s[2][3];  // S^T rows for output halves h = 0, 1; three bf16 parts
  bf16x8_t z[3];     // z in every row; three bf16 parts
};

__device__ __forceinline__ void load_apply_operands(const float* S, const float* z, int g, int m,
                                                    ApplyOperands& op) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 8 * (m >> 2) + 4 * h + (m & 3);
    unsigned part[3][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
      split3_bf16x2(S[(8 * g + 2 * p) * 32 + e], S[(8 * g + 2 * p + 1) * 32 + e], part[0][p], part[1][p],
                    part[2][p]);
#pragma unroll
    for (int k = 0; k < 3; ++k) op.s[h][k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
  }
  unsigned part[3][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    split3_bf16x2(z[8 * g + 2 * p], z[8 * g + 2 * p + 1], part[0][p], part[1][p], part[2][p]);
#pragma unroll
  for (int k = 0; k < 3; ++k) op.z[k] = as_bf16x8(part[k][0], part[k][1], part[k][2], part[k][3]);
}

// One 16-token tile: q holds this lane's 8 raw features; returns the 8 outputs
// packed as bf16 (RNE).
template <bool ROPE>
__device__ __forceinline__ u32x4_t apply_tile(u32x4_t q, const ApplyOperands& op, float eps, f32x4_t c,
                                              f32x4_t sn) {
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  q[0] = relu_bf16x2(q[0]);
  q[1] = relu_bf16x2(q[1]);
  q[2] = relu_bf16x2(q[2]);
  q[3] = relu_bf16x2(q[3]);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, q);

  f32x4_t den = mfma16(op.z[0], b, zero4);
  den = mfma16(op.z[1], b, den);
  den = mfma16(op.z[2], b, den);
  f32x4_t n0, n1;
  if constexpr (!ROPE) {
    n0 = mfma16(op.s[0][0], b, zero4);
    n0 = mfma16(op.s[0][1], b, n0);
    n0 = mfma16(op.s[0][2], b, n0);
    n1 = mfma16(op.s[1][0], b, zero4);
    n1 = mfma16(op.s[1][1], b, n1);
    n1 = mfma16(op.s[1][2], b, n1);
  } else {
    unsigned rq[3][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = bf16lo_to_f32(q[p]);
      const float x1 = bf16hi_to_f32(q[p]);
      split3_bf16x2(rot_lo(x0, x1, c[p], sn[p]), rot_hi(x0, x1, c[p], sn[p]), rq[0][p], rq[1][p], rq[2][p]);
    }
    bf16x8_t b_r[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) b_r[k] = as_bf16x8(rq[k][0], rq[k][1], rq[k][2], rq[k][3]);
    // the six product terms of weight >= 2^-16: hh, hm, mh, hl, lh, mm
    n0 = mfma16(op.s[0][0], b_r[0], zero4);
    n0 = mfma16(op.s[0][0], b_r[1], n0);
    n0 = mfma16(op.s[0][1], b_r[0], n0);
    n0 = mfma16(op.s[0][0], b_r[2], n0);
    n0 = mfma16(op.s[0][2], b_r[0], n0);
    n0 = mfma16(op.s[0][1], b_r[1], n0);
    n1 = mfma16(op.s[1][0], b_r[0], zero4);
    n1 = mfma16(op.s[1][0], b_r[1], n1);
    n1 = mfma16(op.s[1][1], b_r[0], n1);
    n1 = mfma16(op.s[1][0], b_r[2], n1);
    n1 = mfma16(op.s[1][2], b_r[0], n1);
    n1 = mfma16(op.s[1][1], b_r[1], n1);
  }
  const float rinv = 1.0f / (den[0] + eps);
  u32x4_t o;
  o[0] = pack_bf16x2(n0[0] * rinv, n0[1] * rinv);
  o[1] = pack_bf16x2(n0[2] * rinv, n0[3] * rinv);
  o[2] = pack_bf16x2(n1[0] * rinv, n1[1] * rinv);
  o[3] = pack_bf16x2(n1[2] * rinv, n1[3] * rinv);
  return o;
}

// The four 16-token tiles of a wave's 64-token chunk at t0 (this lane: token
// t0 + 16u + m, features 8g .. 8g+7), with cos/sin of its pairs under RoPE.
template <int ROPE>
struct ApplyChunk {
  u32x4_t q[4];
  f32x4_t c[4], sn[4];
};

// Rows at or past n_end read 0; their outputs are not stored.
template <int ROPE, int HEADS>
__device__ __forceinline__ void load_apply_chunk(const char* Qh, int64_t row, int64_t t0, int64_t n_end,
                                                 int lane_off, int tab_off, int m, int g, const Rope& rp,
                                                 const float* rtab, ApplyChunk<ROPE>& ch) {
  const rsrc_t rq = rows_rsrc(Qh, t0, n_end, row);
#pragma unroll
  for (int u = 0; u < 4; ++u) ch.q[u] = load16_stream<HEADS>(rq, lane_off + u * 16 * (int)row);
  if constexpr (ROPE == kRopeTable) {
    // pairs 4g .. 4g+3 of the token at position pos0 + t0 + 16u + m: the same
    // lane offset in a 64-byte table row
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

// A wave's 64-token chunks t0, t0 + step, ... below n_end of one head (step:
// 64 tokens per wave of the workgroup), the first of which `next` already
// holds (loaded before the state operands were fetched): each chunk's loads go
// out before the previous chunk is computed.
template <int ROPE, int HEADS>
__device__ __forceinline__ void apply_stream(const char* Qh, char* Oh, int64_t qrow, int64_t orow, int64_t t0,
                                             int64_t n_end, int q_off, int o_off, int tab_off, int m, int g,
                                             const Rope& rp, const float* rtab, const AxisLane& al,
                                             const ApplyOperands& op, float eps, ApplyChunk<ROPE>& next,
                                             int step = 256) {
  for (; t0 < n_end; t0 += step) {
    const ApplyChunk<ROPE> cur = next;
    if (t0 + step < n_end)
      load_apply_chunk<ROPE, HEADS>(Qh, qrow, t0 + step, n_end, q_off, tab_off, m, g, rp, rtab, next);
    const rsrc_t ro = rows_rsrc(Oh, t0, n_end, orow);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4_t c = cur.c[u], sn = cur.sn[u];
      if constexpr (ROPE == kRopeAxes) rope_axis_row4(rp, rtab, al, rp.pos0 + t0 + 16 * u + m, c, sn);
      store16_nt(ro, o_off + u * 16 * (int)orow, apply_tile<ROPE != 0>(cur.q[u], op, eps, c, sn));
    }
  }
}

template <int ROPE, bool DENSE, int HEADS>
__global__ __launch_bounds__(kThreads* HEADS) void apply_bf16(const u32x4_t* __restrict__ Q, u32x4_t* __restrict__ O,
                                                              Layout lq, Layout lo, StateView sv, int64_t N,
                                                              int64_t L, int C, int64_t total, int64_t La, float eps,
                                                              Rope rp, int64_t BH) {
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads * HEADS);
  if constexpr (ROPE == kRopeAxes) __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wg >> 2;
  const int w = wg & 3;
  const int m = lane & 15;
  const int g = lane >> 4;
  const AxisLane al = axis_lane(rp, g);  // axis form only
  const int64_t qrow = DENSE ? 64 : lq.token * 2, orow = DENSE ? 64 : lo.token * 2;  // bytes between tokens
  const int q_off = m * (int)qrow + g * 16;                // features 8g .. 8g+7 of tile row m
  const int o_off = m * (int)orow + g * 16;
  const int tab_off = m * 64 + g * 16;
  int64_t f_begin, f_end;
  if constexpr (HEADS == 2) {
    const int64_t units = (BH + 1) / 2;
    const int64_t u = blockIdx.x % units;
    f_begin = u * N + (int64_t)(blockIdx.x / units) * La;
    f_end = (f_begin + La < (u + 1) * N) ? f_begin + La : (u + 1) * N;
  } else {
    f_begin = (int64_t)blockIdx.x * La;
    f_end = (f_begin + La < total) ? f_begin + La : total;
  }

  // the range is processed in segments that stay inside one head and chunk
  for (int64_t f = f_begin; f < f_end;) {
    const int64_t unit = f / N;
    const int64_t n_begin = f - unit * N;
    const int c = (int)(n_begin / L);
    const int64_t c_end = ((int64_t)c + 1) * L < N ? ((int64_t)c + 1) * L : N;
    const int64_t n_end = (f_end - unit * N < c_end) ? f_end - unit * N : c_end;
    f = unit * N + n_end;
    const int64_t bh = unit * HEADS + half;
    if (bh >= BH) continue;
    const char* Qh = reinterpret_cast<const char*>(Q) + lq.base(bh) * 2;
    char* Oh = reinterpret_cast<char*>(O) + lo.base(bh) * 2;

    // the first chunk's loads go out before the state operands are fetched,
    // and each chunk's loads before the previous chunk is computed
    int64_t t0 = n_begin + 64 * w;
    ApplyChunk<ROPE> next;
    if (t0 < n_end) load_apply_chunk<ROPE, HEADS>(Qh, qrow, t0, n_end, q_off, tab_off, m, g, rp, rtab, next);
    ApplyOperands op;
    const int64_t sc = bh * C + c;
    load_apply_operands(sv.s_base + sc * sv.s_stride, sv.z_base + sc * sv.z_stride, g, m, op);

    apply_stream<ROPE, HEADS>(Qh, Oh, qrow, orow, t0, n_end, q_off, o_off, tab_off, m, g, rp, rtab, al, op, eps,
                              next);
  }
}

// ---------------------------------------------------------------------------
// Whole-head forward (bf16, dense layouts): state pass and apply in one launch
// ---------------------------------------------------------------------------
// When each head is one chunk taken by one workgroup (short sequences over
// many heads), the workgroup that sums a head's state can apply it as well:
// no partial, no finalize, no second launch.  Both halves are the passes' own
// code -- the same four waves and chunk order, the same wave-tile sum, the
// same apply tiles -- so the results are those of the two-launch path bit for
// bit.  Each wave's first query chunk is loaded before the state work starts.
// The full-table RoPE form is not taken here: its prefetched angle rows would
// sit in registers through the state pass.
template <int ROPE>
__global__ __launch_bounds__(kThreads) void forward_whole_bf16(const u32x4_t* __restrict__ K,
                                                               const u32x4_t* __restrict__ V,
                                                               const u32x4_t* __restrict__ Q, u32x4_t* __restrict__ O,
                                                               Layout lin, Layout lo, Rope rp, StateArgs a, int64_t N,
                                                               float eps) {
  static_assert(ROPE != kRopeTable, "the full-table form takes the two-launch path");
  __shared__ float red[4][kStateElems];
  __shared__ float angles[ROPE ? 4 : 1][ROPE ? kAngTile : 1];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const char* Kh = reinterpret_cast<const char*>(K) + lin.base(bh) * 2;
  const char* Vh = reinterpret_cast<const char*>(V) + lin.base(bh) * 2;
  const char* Qh = reinterpret_cast<const char*>(Q) + lin.base(bh) * 2;
  char* Oh = reinterpret_cast<char*>(O) + lo.base(bh) * 2;
  const int lane_off = n * 64 + g * 16;  // features 8g .. 8g+7 of tile row n (64-byte rows)
  const int64_t t0 = 64 * w;

  ApplyChunk<ROPE> next;
  if (t0 < N) load_apply_chunk<ROPE, 1>(Qh, 64, t0, N, lane_off, lane_off, n, g, rp, rtab, next);

  f32x4_t acc[2][2], accz[2];
  state_accumulate<ROPE, 1>(Kh, Vh, 64, t0, N, rp, rtab, angles[ROPE ? w : 0], g, n, acc, accz);
  state_to_lds(acc, accz, red[w], g, n);
  __syncthreads();
  sum_wave_tiles(red, tid);
  __syncthreads();
  // the head's state: the carried one plus this sequence's, committed when
  // asked, and kept in red[1] for the apply
  for (int idx = tid; idx < kStateElems; idx += kThreads) {
    const float x = carried(a, bh, idx) + red[0][idx];
    red[1][idx] = x;
    if (a.kv_out) commit(a, bh, idx, x);
  }
  __syncthreads();

  ApplyOperands op;
  load_apply_operands(red[1], red[1] + 1024, g, n, op);
  const AxisLane al = axis_lane(rp, g);  // axis form only
  apply_stream<ROPE, 1>(Qh, Oh, 64, 64, t0, N, lane_off, lane_off, lane_off, n, g, rp, rtab, al, op, eps, next);
}

// ---------------------------------------------------------------------------
// Apply with the finalize folded in (bf16, dense, one chunk; no RoPE or per-axis)
// ---------------------------------------------------------------------------
// Two launches per call instead of three: the state pass (items dealt XCD by
// XCD) leaves each head's Pc partials, and each of the head's P apply
// workgroups of WAVES waves, on the same XCD, sums them itself onto the carried
// state, in split order as the finalize does, before applying the state to
// its 1/P of the queries.  The state, the saved chunk state (part 0) and the
// commit (part P - 1) are the finalize's bit for bit, and the apply tiles are
// apply_bf16's, so the results are the three-launch path's.
//
// Commit.  When kv_out may alias kv_in, parts 0 .. P-2 publish per call that
// they have read the carried state (flags[bh * P + p] = epoch, a number the
// host takes fresh for every call), and part P - 1 waits for those words
// before it stores.  Its siblings have lower block numbers on the same XCD,
// so they were dispatched before it and every wait ends; the spin is bounded
// as well.
constexpr int kFoldMaxSplits = 16;
constexpr int kFoldSpinLimit = 1 << 22;

struct FoldArgs {
  int64_t Na;        // queries per part (a multiple of 64)
  unsigned* flags;   // [BH][P] arrival words (commit over a carried state), else null
  unsigned epoch;    // this call's number
  int P;             // workgroups per head
};

// ROPE: none or the per-axis form (its tables staged in LDS, as apply_bf16
// stages them).
// 16 waves per CU: at most 128 VGPRs (the second bound is waves per SIMD).
template <int WAVES, int ROPE>
__global__ __launch_bounds__(64 * WAVES, 4) void apply_fold_bf16(const u32x4_t* __restrict__ Q, u32x4_t* __restrict__ O,
                                                              Layout lq, Layout lo, StateArgs a, FoldArgs f, int64_t BH,
                                                              float eps, Rope rp) {
  static_assert(ROPE != kRopeTable, "the full-table form takes the three-launch path");
  constexpr int kFoldThreads = 64 * WAVES;
  __shared__ float st[kStateElems];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  const int slot = blockIdx.x / kXcdCount;
  const int64_t bh = blockIdx.x % kXcdCount + (int64_t)kXcdCount * (slot / f.P);
  const int p = slot % f.P;
  if (bh >= BH) return;
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kFoldThreads);
  if constexpr (ROPE == kRopeAxes) __syncthreads();
  const int64_t N = a.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15;
  const int g = lane >> 4;
  const char* Qh = reinterpret_cast<const char*>(Q) + lq.base(bh) * 2;
  char* Oh = reinterpret_cast<char*>(O) + lo.base(bh) * 2;
  const int lane_off = m * 64 + g * 16;

  // this part's queries: each wave's first chunk goes out first
  const int64_t q_begin = (int64_t)p * f.Na;
  const int64_t q_end = (q_begin + f.Na < N) ? q_begin + f.Na : N;
  const int64_t t0 = q_begin + 64 * wave;
  ApplyChunk<ROPE> next;
  if (t0 < q_end) load_apply_chunk<ROPE, 1>(Qh, 64, t0, q_end, lane_off, lane_off, m, g, rp, rtab, next);

  // the head's state: the carried one plus the partials in split order; the
  // loads go out together (those past the last partial re-read it, unused)
  const float* src = a.partials + bh * a.Pc * kStateElems;
  for (int idx = tid; idx < kStateElems; idx += kFoldThreads) {
    float v[kFoldMaxSplits];
#pragma unroll
    for (int u = 0; u < kFoldMaxSplits; ++u) v[u] = src[(int64_t)min(u, a.Pc - 1) * kStateElems + idx];
    float acc = carried(a, bh, idx);
#pragma unroll
    for (int u = 0; u < kFoldMaxSplits; ++u)
      if (u < a.Pc) acc += v[u];
    st[idx] = acc;
    if (p == 0) a.states[bh * kStateElems + idx] = acc;
  }
  __syncthreads();
  // every lane has used its carried values: say so to the committing part
  if (f.flags && p != f.P - 1 && tid == 0)
    __hip_atomic_store(f.flags + bh * f.P + p, f.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  ApplyOperands op;
  load_apply_operands(st, st + 1024, g, m, op);
  const AxisLane al = axis_lane(rp, g);
  apply_stream<ROPE, 1>(Qh, Oh, 64, 64, t0, q_end, lane_off, lane_off, lane_off, m, g, rp, rtab, al, op, eps, next,
                        64 * WAVES);

  if (a.kv_out && p == f.P - 1) {
    if (f.flags && tid == 0) {
      for (int u = 0; u < f.P - 1; ++u) {
        for (int spin = 0; spin < kFoldSpinLimit; ++spin) {
          if (__hip_atomic_load(f.flags + bh * f.P + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == f.epoch)
            break;
          __builtin_amdgcn_s_sleep(2);
        }
      }
    }
    __syncthreads();
    for (int idx = tid; idx < kStateElems; idx += kFoldThreads) commit(a, bh, idx, st[idx]);
  }
}

// ---------------------------------------------------------------------------
// fp32 apply pass (VALU): thread = (token, 4 output features)
// ---------------------------------------------------------------------------
// Workgroup (bh, c, tile) applies tokens [c*L + tile*Lt, ...) of chunk c.
template <int ROPE>
__global__ __launch_bounds__(kThreads) void apply_f32(const float* __restrict__ Q, float* __restrict__ O,
                                                      Layout lq, Layout lo, StateView sv, int64_t N, int64_t L,
                                                      int C, int T, int64_t Lt, float eps, Rope rp) {
  __shared__ float sS[kD][kD];
  __shared__ float sz[kD];
  __shared__ __attribute__((aligned(16))) float rtab[ROPE == kRopeAxes ? 2 * kMaxAxisTab : 1];
  rope_stage<ROPE>(rp, rtab, threadIdx.x, kThreads);
  const int64_t bh = blockIdx.x / ((int64_t)C * T);
  const int r = (int)(blockIdx.x % ((int64_t)C * T));
  const int c = r / T;
  const int tile = r % T;
  const int64_t c_end = ((int64_t)c + 1) * L < N ? ((int64_t)c + 1) * L : N;
  const int64_t n_begin = (int64_t)c * L + (int64_t)tile * Lt;
  const int64_t n_end = (n_begin + Lt < c_end) ? n_begin + Lt : c_end;
  const int t = threadIdx.x;
  const int64_t sc = bh * C + c;
  for (int idx = t; idx < 1024; idx += kThreads) sS[idx >> 5][idx & 31] = sv.s_base[sc * sv.s_stride + idx];
  if (t < kD) sz[t] = sv.z_base[sc * sv.z_stride + t];
  __syncthreads();
  const int tl = t >> 3;
  const int e0 = (t & 7) * 4;
  for (int64_t tok = n_begin + tl; tok < n_end; tok += 32) {
    const float* qrow = Q + lq.base(bh) + tok * lq.token;
    float pq[kD], pr[kD];
#pragma unroll
    for (int d = 0; d < kD; ++d) pq[d] = fmaxf(qrow[d], 0.f);
    float den = 0.f;
#pragma unroll
    for (int d = 0; d < kD; ++d) den = fmaf(pq[d], sz[d], den);
    den += eps;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      if constexpr (ROPE) {
        float c, sn;
        rope_pair<ROPE>(rp, rtab, rp.pos0 + tok, p, c, sn);
        pr[2 * p] = rot_lo(pq[2 * p], pq[2 * p + 1], c, sn);
        pr[2 * p + 1] = rot_hi(pq[2 * p], pq[2 * p + 1], c, sn);
      } else {
        pr[2 * p] = pq[2 * p];
        pr[2 * p + 1] = pq[2 * p + 1];
      }
    }
    float num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < kD; ++d) {
#pragma unroll
      for (int c = 0; c < 4; ++c) num[c] = fmaf(pr[d], sS[d][e0 + c], num[c]);
    }
    float* orow = O + lo.base(bh) + tok * lo.token + e0;
#pragma unroll
    for (int c = 0; c < 4; ++c) orow[c] = num[c] / den;
  }
}

}  // namespace la
