/*
 * sana_linattn.h -- C ABI of SANA's ReLU linear attention on MI355X (gfx950).
 *
 * The operation (phi = ReLU on queries and keys, D = head width):
 *
 *   per (batch b, head h):  S = sum_j phi(K_j)^T V_j   (D x D, row d = key feature,
 *                                                        column e = value feature)
 *                           z = sum_j phi(K_j)         (D)
 *   per token i:            O_i = phi(Q_i) . S / (phi(Q_i) . z + eps)
 *
 * Sources (page title, section):
 *   - "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion
 *     Transformers" (research note), "Model architecture" item 2) Linear DiT:
 *     ReLU linear attention whose shared sums sum ReLU(K_j)^T V_j and
 *     sum ReLU(K_j) are computed once and reused by every query.
 *   - "SANA-Video: Efficient Video Generation with Block Linear Diffusion
 *     Transformer" (paper notes), section 2.1 (precomputed state, O(D^2) per
 *     token), 2.2 (RoPE applied after the ReLU, left out of the denominator),
 *     2.3 (constant-memory causal state: D x D state sum plus D x 1 key sum)
 *     and 4 (block inference: denoising steps read the cache, a final pass on
 *     the clean chunk commits it).
 *   - SANA-Video news article (mjgaz.cn), "Design details": later blocks see
 *     earlier ones, never the reverse; KV1 + KV2 -> KV1-2 ... -> KVsum, and
 *     each block sums KVsum with its own KV.
 *
 * The pages print no normalisation formula (it is lost in the extraction); eps
 * is added after the dot product, as written above.  There is no 1/sqrt(D)
 * scale.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Layout     Q, K, V, O are contiguous [B][H][N][D] arrays, D innermost, in
 *              device memory, each 16-byte aligned (the *_strided entry
 *              points take other layouts, see sana_layout).  kv state is [B][H][D][D]
 *              float (row = key feature, column = value feature), ksum state
 *              is [B][H][D] float, both in device memory, 4-byte aligned.
 *   Dtype      One dtype for Q, K, V and O (sana_dtype).  States, RoPE tables
 *              and all accumulation are fp32.  bf16 results are rounded to
 *              nearest-even once, at the store.
 *   D          Only D = 32 (the head width of Sana-0.6B and Sana-1.6B) has
 *              kernels; any other positive D returns SANA_ERR_UNSUPPORTED.
 *   Ownership  The caller allocates and owns every buffer, the workspace
 *              included.  The library never allocates, frees or synchronises;
 *              it keeps no state between calls and is re-entrant.
 *   Streams    Work is enqueued asynchronously on `hip_stream` (a
 *              hipStream_t; NULL = the default stream) and the call returns
 *              without waiting for it.
 *   Workspace  `ws` is device scratch of at least
 *              sana_linattn_workspace_bytes(...) bytes, 256-byte aligned, with
 *              no initial contents required.  The part of it a call writes
 *              (its workspace_bytes) may overlap none of the call's tensors,
 *              states or RoPE tables (SANA_ERR_INVALID).  Calls that overlap
 *              in time must use different workspaces.
 *   Errors     Arguments are checked before anything is enqueued; on error
 *              nothing is launched and a negative sana_status is returned:
 *                SANA_ERR_INVALID      NULL pointer where work exists, B, H or
 *                                      N negative, chunk <= 0, D <= 0, unknown dtype,
 *                                      non-finite or negative eps, misaligned
 *                                      pointer, O overlapping Q/K/V, a
 *                                      workspace overlapping a buffer of the
 *                                      call, RoPE rows out of the table, size
 *                                      overflow
 *                SANA_ERR_UNSUPPORTED  D != 32
 *                SANA_ERR_WORKSPACE    ws NULL or ws_bytes too small
 *                SANA_ERR_HIP          a launch reported a HIP error
 *   Empty      B*H*N == 0 is a no-op returning SANA_OK (pointers unchecked).
 *   RoPE       A NULL `rope` means no rotation.  Otherwise token n of every
 *              head (global position pos_offset + n) rotates the interleaved
 *              pairs (2p, 2p+1) of phi(Q_n) and phi(K_n) by the angle whose
 *              cosine and sine are cos[pos][p] and sin[pos][p]:
 *              (x0, x1) -> (x0 c - x1 s, x0 s + x1 c).  The rotation enters
 *              the numerator only; z and the denominator stay un-rotated.
 */
#ifndef SANA_LINATTN_H
#define SANA_LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SANA_OK = 0,
    SANA_ERR_INVALID = -1,
    SANA_ERR_UNSUPPORTED = -2,
    SANA_ERR_WORKSPACE = -3,
    SANA_ERR_HIP = -4
} sana_status;

typedef enum {
    SANA_DT_F32 = 0,
    SANA_DT_BF16 = 1
} sana_dtype;

/* RoPE angles ("SANA-Video" paper notes, section 2.2: applied after the ReLU,
 * numerator only).  Pair p of a token rotates features (2p, 2p+1) by the angle
 * whose cosine and sine the tables give for the token's position
 * pos_offset + n; positions pos_offset .. pos_offset+N-1 must lie in
 * [0, n_pos).  Two forms:
 *   full tables (grid and pairs all 0): cos, sin are device arrays
 *     [n_pos][D/2] fp32, 16-byte aligned, pair p of position pos at [pos][p];
 *   per-axis tables of a 3D RoPE (grid = {T, Hl, Wl}, all > 0; section 3
 *     Stage 2): position pos is the latent point pos = (t*Hl + h)*Wl + w,
 *     n_pos = T*Hl*Wl; the first pairs[0] pairs turn with t, the next
 *     pairs[1] with h, the last pairs[2] with w (even counts summing to D/2),
 *     by angles that depend on that coordinate only.  cos, sin are device
 *     arrays (4-byte aligned) holding [T][pairs[0]], then [Hl][pairs[1]],
 *     then [Wl][pairs[2]] fp32 back to back, at most 1024 floats each;
 *     Hl*Wl < 2^20.  Each workgroup copies them to LDS instead of streaming a
 *     [n_pos][D/2] table per head; with equal angle values both forms give
 *     identical results. */
typedef struct {
    const float* cos;
    const float* sin;
    int64_t n_pos;
    int64_t pos_offset;
    int32_t grid[3];
    int32_t pairs[3];
} sana_rope;

/* Element strides of a [B][H][N][D] tensor view, D contiguous: token n of head
 * h in batch b starts at element b*batch + h*head + n*token.  Examples (D = 32):
 *   contiguous [B][H][N][D]             {H*N*D, N*D, D}   (what NULL means)
 *   [B][N][H][D]                        {N*H*D, D, H*D}
 *   q (k, v) of a packed [B][N][3][H][D] projection output: {N*3*H*D, D, 3*H*D},
 *   with k and v at element offsets H*D and 2*H*D from q.
 * Requirements: strides >= 0, token >= D; batch, head and token strides times
 * the element size multiples of 16 bytes; token row stride at most 16 MiB.
 * Input views may alias one another (as in the packed example); an output view
 * must map distinct (b, h, n, d) to distinct elements (nested strides), and an
 * output's address span (first to last element) must not overlap any other
 * tensor's span or the state buffers.  Violations return SANA_ERR_INVALID. */
typedef struct {
    int64_t batch;
    int64_t head;
    int64_t token;
} sana_layout;

/* Bytes of device workspace that forward, state_update and block_forward need
 * for these sizes (0 when B*H*N == 0).  Pure host function, no HIP call.
 * Returns 0 as well for invalid sizes; the entry points then reject them. */
size_t sana_linattn_workspace_bytes(int B, int H, int64_t N, int D, int dtype, int has_rope);

/* Kernel launches that one call of sana_linattn_forward (chunk = N),
 * sana_linattn_block_forward (chunk = N) or sana_linattn_block_causal (chunk)
 * makes for these sizes, for tools that report per-kernel figures.  1 when
 * every head is one chunk taken by one workgroup (see the geometry in the
 * implementation: at least 128 heads of at most 1024 tokens, or heads of at
 * most 256) with bf16 data in dense layouts and no full-table RoPE: the state
 * pass and the apply then run in one launch.  Otherwise 2 (state pass, apply)
 * or 3 (with the finalize, when a head has several partials).  rope_form: 0
 * none, 1 full tables, 2 per-axis tables; dense: 1 when Q, K, V and O are
 * contiguous [B, H, N, D].  Pure host function, no HIP call; returns 0 when
 * the call would launch nothing (B*H*N == 0) or for invalid arguments. */
int sana_linattn_forward_launches(int B, int H, int64_t N, int64_t chunk, int D, int dtype, int rope_form,
                                  int dense);

/* Non-causal forward ("Sana" research note, Model architecture item 2;
 * "SANA-Video" paper notes 2.1, 2.2):
 *   O_i = phi~(Q_i) . S / (phi(Q_i) . z + eps) with S, z summed over all N
 *   tokens of the same (b, h).  phi~ is phi rotated by `rope` (positions
 *   pos_offset .. pos_offset+N-1), or phi itself when rope is NULL.
 * q, k, v: inputs [B][H][N][D]; o: output, same shape and dtype, must not
 * overlap q, k or v. */
int sana_linattn_forward(const void* q, const void* k, const void* v, void* o,
                         int B, int H, int64_t N, int D, int dtype, float eps,
                         const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* Commit N tokens into a carried state, without outputs ("SANA-Video" paper
 * notes 2.3 and 4; news article "Design details", KV1 + KV2 -> KV1-2):
 *   kv_state[b][h]   += sum_j phi~(K_j)^T V_j
 *   ksum_state[b][h] += sum_j phi(K_j)
 * k, v: inputs [B][H][N][D]; kv_state, ksum_state: read and updated in place.
 * With rope, key j is rotated at position pos_offset + j; ksum never is. */
int sana_linattn_state_update(const void* k, const void* v, float* kv_state, float* ksum_state,
                              int B, int H, int64_t N, int D, int dtype,
                              const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* The key/value projection and the state update in one pass ("Sana" research
 * note, "Infra": ReLU(K)^T V fused into the QKV projection, there in an INT8
 * engine).  Per batch b and head h, with K = x[b] W_k[h]^T and V = x[b] W_v[h]^T
 * each rounded to bf16 as a bf16 projection would store them:
 *   kv_state[b][h]   += sum_j phi~(K_j)^T V_j
 *   ksum_state[b][h] += sum_j phi(K_j)
 * exactly what sana_linattn_state_update adds for that K and V, which are
 * never written to memory.  With rope (either form of sana_rope), key j of
 * every batch is rotated at position pos_offset + j after the ReLU, in the
 * numerator state only ("SANA-Video" paper notes 2.2); NULL: no rotation.
 * x: input activations [B][N][C] bf16 (channels innermost).  w_k, w_v: weights
 * [H*D][C] bf16, row h*D + d holding output feature d of head h (the layout of
 * a linear layer's weight, or of the key or value rows of a fused QKV weight).
 * All three 16-byte aligned in device memory.  kv_state [B][H][D][D],
 * ksum_state [B][H][D]: fp32, read and updated in place (zero them first for
 * the state of these N tokens alone).  C must be a positive multiple of 32, at
 * most 65536 (else SANA_ERR_INVALID); only dtype SANA_DT_BF16 and D = 32 have
 * kernels (else SANA_ERR_UNSUPPORTED).  The products accumulate in
 * fp32.  ws: at least sana_linattn_project_state_workspace_bytes(...) bytes.
 * B*H*N = 0 leaves the states unchanged. */
int sana_linattn_project_state(const void* x, const void* w_k, const void* w_v, float* kv_state,
                               float* ksum_state, int B, int H, int64_t N, int C, int D, int dtype,
                               const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* Workspace bytes for sana_linattn_project_state with these sizes (0 when there
 * is no work or the sizes are invalid).  Pure host function. */
size_t sana_linattn_project_state_workspace_bytes(int B, int H, int64_t N, int C, int D, int dtype);

/* The query projection and the apply step in one pass (the other half of the
 * projection fusion the "Sana" research note lists under "Infra").  Per batch
 * b and head h, with Q = x[b] W_q[h]^T rounded to bf16 as a bf16 projection
 * would store it (never written to memory):
 *   O_i = phi~(Q_i) . S / (phi(Q_i) . z + eps),  S = kv_state[b][h], z = ksum_state[b][h]
 * exactly what sana_linattn_apply computes for that Q ("SANA-Video" paper
 * notes 2.1, 2.2: RoPE, if any, in the numerator only, query i at position
 * pos_offset + i).  x: [B][N][C] bf16; w_q: [H*D][C] bf16 (row h*D + d = query
 * feature d of head h), both 16-byte aligned; o: bf16 outputs [B][H][N][D]
 * through the view `out` (NULL: contiguous; e.g. [B][N][H][D]), overlapping
 * no input; kv_state [B][H][D][D], ksum_state [B][H][D]: fp32, read only (for
 * example from sana_linattn_project_state).  eps >= 0 and finite.
 * SANA_ERR_INVALID: negative sizes, C not a positive multiple of 32 or above
 * 65536, a NULL or misaligned pointer, o overlapping an input, a bad view, bad
 * eps, or RoPE tables shorter than pos_offset + N.  SANA_ERR_UNSUPPORTED: a
 * dtype other than bf16 or D other than 32.  No workspace.  B*H*N = 0 is a
 * no-op that touches nothing. */
int sana_linattn_project_apply(const void* x, const void* w_q, void* o, const sana_layout* out,
                               const float* kv_state, const float* ksum_state, int B, int H, int64_t N, int C,
                               int D, int dtype, float eps, const sana_rope* rope, void* hip_stream);

/* sana_linattn_forward with Q, K, V read through the view `in` and O written
 * through `out` (NULL: contiguous), e.g. straight from a [B][N][3][H][D] QKV
 * projection output, with no relayout copy.  Everything else as for
 * sana_linattn_forward; the workspace size does not depend on the layout. */
int sana_linattn_forward_strided(const void* q, const void* k, const void* v, void* o,
                                 const sana_layout* in, const sana_layout* out,
                                 int B, int H, int64_t N, int D, int dtype, float eps,
                                 const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* One chunk of block-causal attention ("SANA-Video" paper notes 2.3 and 4;
 * news article "Design details"): the chunk's queries see the state carried
 * from earlier chunks plus every token of the chunk itself.
 *   S_new = kv_in + sum_{j in chunk} phi~(K_j)^T V_j,   z_new = ksum_in + sum phi(K_j)
 *   O_i   = phi~(Q_i) . S_new / (phi(Q_i) . z_new + eps)
 * kv_in/ksum_in: state of earlier chunks, or both NULL for a zero state (first
 * chunk).  kv_out/ksum_out: where S_new/z_new are committed, or both NULL to
 * leave the carried state untouched (a denoising step that only reads the
 * cache).  kv_out may equal kv_in and ksum_out may equal ksum_in (in-place
 * commit); no other overlap between state buffers and q/k/v/o is allowed.
 * With rope, the chunk's token n sits at global position pos_offset + n. */
int sana_linattn_block_forward(const void* q, const void* k, const void* v, void* o,
                               const float* kv_in, const float* ksum_in,
                               float* kv_out, float* ksum_out,
                               int B, int H, int64_t N, int D, int dtype, float eps,
                               const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* Bytes of the static scratch array behind sana_linattn_block_forward_noalloc
 * (one copy per GPU, held until the process ends). */
#define SANA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* sana_linattn_block_forward for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and kernels as sana_linattn_block_forward (bit for bit
 * the same outputs and commits), with no workspace argument: its scratch
 * (split partials and the chunk state) lives in a file-scope device array of
 * SANA_NOALLOC_SCRATCH_BYTES, whose address on the current device is looked
 * up once, on the first call on that device (so make that first call outside
 * graph capture).  The call allocates and frees nothing, copies, clears and
 * synchronises nothing.  A call that needs more scratch than the array holds
 * (sana_linattn_workspace_bytes(B, H, N, ...) > SANA_NOALLOC_SCRATCH_BYTES,
 * i.e. more than about 1900 heads B*H) returns SANA_ERR_WORKSPACE before
 * anything is launched.  Every call on one GPU shares that GPU's array and no
 * call needs its earlier contents; calls that overlap on one GPU (two streams
 * at once) race on it and must not be made.  hip_stream must belong to the
 * current device.  A failed address lookup returns SANA_ERR_HIP.  Other
 * arguments, layouts and errors: as sana_linattn_block_forward. */
int sana_linattn_block_forward_noalloc(const void* q, const void* k, const void* v, void* o,
                                       const float* kv_in, const float* ksum_in,
                                       float* kv_out, float* ksum_out,
                                       int B, int H, int64_t N, int D, int dtype, float eps,
                                       const sana_rope* rope, void* hip_stream);

/* sana_linattn_block_forward through layout views (see sana_linattn_forward_strided). */
int sana_linattn_block_forward_strided(const void* q, const void* k, const void* v, void* o,
                                       const sana_layout* in, const sana_layout* out,
                                       const float* kv_in, const float* ksum_in,
                                       float* kv_out, float* ksum_out,
                                       int B, int H, int64_t N, int D, int dtype, float eps,
                                       const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* A whole sequence in block-causal chunks, in one call ("SANA-Video" paper
 * notes 2.3 and section 3's block-wise training; news article "Design
 * details": later blocks see earlier ones, never the reverse, and each block
 * sums KVsum with its own KV).  Token n of a head belongs to chunk
 * c(n) = n / chunk (the last chunk may be shorter); with
 *   S_c = kv_in + sum_{j : c(j) <= c} phi~(K_j)^T V_j,  z_c = ksum_in + sum phi(K_j)
 *   O_n = phi~(Q_n) . S_{c(n)} / (phi(Q_n) . z_{c(n)} + eps)
 * i.e. the same result as calling block_forward chunk after chunk with an
 * in-place commit, for when every chunk's Q, K, V is available at once (block
 * training, re-encoding a sequence).  kv_in/ksum_in: state before the first
 * chunk, or both NULL for zero; kv_out/ksum_out: where the state after the
 * last chunk is committed, or both NULL (may equal kv_in/ksum_in).  chunk must
 * be positive; chunk >= N is one chunk (the same as block_forward).  With
 * rope, token n sits at global position pos_offset + n.  Workspace:
 * sana_linattn_block_causal_workspace_bytes. */
int sana_linattn_block_causal(const void* q, const void* k, const void* v, void* o,
                              const float* kv_in, const float* ksum_in,
                              float* kv_out, float* ksum_out,
                              int B, int H, int64_t N, int64_t chunk, int D, int dtype, float eps,
                              const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* sana_linattn_block_causal through layout views (see sana_linattn_forward_strided). */
int sana_linattn_block_causal_strided(const void* q, const void* k, const void* v, void* o,
                                      const sana_layout* in, const sana_layout* out,
                                      const float* kv_in, const float* ksum_in,
                                      float* kv_out, float* ksum_out,
                                      int B, int H, int64_t N, int64_t chunk, int D, int dtype, float eps,
                                      const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* Workspace bytes for sana_linattn_block_causal with these sizes (0 when
 * B*H*N == 0 or the sizes are invalid).  Pure host function. */
size_t sana_linattn_block_causal_workspace_bytes(int B, int H, int64_t N, int64_t chunk, int D, int dtype,
                                                 int has_rope);

/* Backward of sana_linattn_block_causal (and, with chunk >= N, of
 * sana_linattn_forward).  The "Sana" research note (Infra) fuses the linear
 * attention's forward and backward into kernels, and "SANA-Video" paper notes
 * 3 train the block-causal model; the pages print no gradient formulas, so
 * these are the chain rule through the forward above, for
 *   L = sum_n dout_n . O_n + <dkv_out, S_last> + dksum_out . z_last
 * with S_last/z_last the state after the last chunk (what a commit stores):
 *   den_n = phi(Q_n).z_c + eps,  dnum_n = dout_n / den_n,
 *   dden_n = -(dout_n . phi~(Q_n) S_c) / den_n^2           (c = c(n))
 *   dq_n = [Q_n > 0] (R_n^T S_c dnum_n + z_c dden_n)
 *   G_c  = dkv_out + sum_{c' >= c} sum_{n in c'} phi~(Q_n) dnum_n^T   (Gz_c with phi(Q_n) dden_n)
 *   dk_n = [K_n > 0] (R_n^T G_c V_n + Gz_c),   dv_n = G_c^T phi~(K_n)
 *   dkv_in = G_0, dksum_in = Gz_0
 * (ReLU'(0) = 0; R_n: the RoPE rotation at position pos_offset + n, identity
 * without rope).  The chunk states S_c are recomputed from k, v and kv_in.
 * q, k, v, dout: inputs [B][H][N][D] of one dtype; dq, dk, dv: outputs of the
 * same shape and dtype, overlapping nothing.  kv_in/ksum_in: state the forward
 * started from, or both NULL (zero).  dkv_out/dksum_out: gradient reaching the
 * committed final state, or both NULL (zero).  dkv_in/dksum_in: where the
 * gradient of kv_in/ksum_in is stored, or both NULL; they may equal
 * dkv_out/dksum_out (in place), no other overlap is allowed.  Chaining: the
 * backward of a chunk-by-chunk block_forward loop is this call chunk by chunk
 * in reverse order, each passing its dkv_in on as the previous chunk's
 * dkv_out.  N = 0 writes nothing.  Workspace:
 * sana_linattn_backward_workspace_bytes.  Errors as for block_causal. */
int sana_linattn_backward(const void* q, const void* k, const void* v, const void* dout,
                          void* dq, void* dk, void* dv,
                          const float* kv_in, const float* ksum_in,
                          const float* dkv_out, const float* dksum_out,
                          float* dkv_in, float* dksum_in,
                          int B, int H, int64_t N, int64_t chunk, int D, int dtype, float eps,
                          const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* sana_linattn_backward with q, k, v, dout read through the view `in` and
 * dq, dk, dv written through `out` (NULL: contiguous); see
 * sana_linattn_forward_strided.  dq, dk, dv each need a view of their own
 * (distinct buffers or disjoint spans). */
int sana_linattn_backward_strided(const void* q, const void* k, const void* v, const void* dout,
                                  void* dq, void* dk, void* dv,
                                  const sana_layout* in, const sana_layout* out,
                                  const float* kv_in, const float* ksum_in,
                                  const float* dkv_out, const float* dksum_out,
                                  float* dkv_in, float* dksum_in,
                                  int B, int H, int64_t N, int64_t chunk, int D, int dtype, float eps,
                                  const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* sana_linattn_backward_strided without recomputing the chunk states: ws must
 * be the workspace of the forward call these gradients belong to, unchanged
 * since (sana_linattn_forward or _strided for chunk = N, or
 * sana_linattn_block_causal, block_forward or their _strided forms with this
 * chunk, on tensors of the same B, H, N, dtype and RoPE).  Every such call
 * leaves its chunk states, carried state included, in the workspace; this call
 * reads them instead of running the state pass again (the carried state is
 * therefore not an argument) and overwrites them, so one forward serves one
 * backward.  The workspace size is the same for both calls.  Results equal
 * sana_linattn_backward's bit for bit.  Other arguments and errors as for
 * sana_linattn_backward_strided.  For the callers that keep a forward's
 * context for its backward, as autograd does. */
int sana_linattn_backward_saved(const void* q, const void* k, const void* v, const void* dout,
                                void* dq, void* dk, void* dv,
                                const sana_layout* in, const sana_layout* out,
                                const float* dkv_out, const float* dksum_out,
                                float* dkv_in, float* dksum_in,
                                int B, int H, int64_t N, int64_t chunk, int D, int dtype, float eps,
                                const sana_rope* rope, void* ws, size_t ws_bytes, void* hip_stream);

/* Backward of sana_linattn_state_update (the key side of every backward):
 * given the gradient (dkv, dksum) reaching an updated state, the gradients of
 * the keys and values that were added into it.  With
 * L = <dkv, S> + dksum . z, S = sum_j phi~(K_j)^T V_j, z = sum_j phi(K_j)
 * ("SANA-Video" paper notes 2.2-2.3):
 *   dk_j = [K_j > 0] (R_j^T dkv V_j + dksum),   dv_j = dkv^T phi~(K_j)
 * (R_j: the RoPE rotation at position pos_offset + j, identity without rope;
 * the state's own gradient passes through unchanged and is not written).
 * k, v: inputs [B][H][N][D]; dkv [B][H][D][D], dksum [B][H][D]: fp32, read
 * only; dk, dv: outputs of k's shape and dtype, overlapping nothing.  No
 * workspace.  N = 0 writes nothing. */
int sana_linattn_state_update_backward(const void* k, const void* v, const float* dkv, const float* dksum,
                                       void* dk, void* dv, int B, int H, int64_t N, int D, int dtype,
                                       const sana_rope* rope, void* hip_stream);

/* Workspace bytes for sana_linattn_backward with these sizes (0 when B*H*N == 0
 * or the sizes are invalid).  Pure host function. */
size_t sana_linattn_backward_workspace_bytes(int B, int H, int64_t N, int64_t chunk, int D, int dtype,
                                             int has_rope);

/* Apply a given state to queries, without changing it ("SANA-Video" paper
 * notes 2.1: the precomputed sum is reused by every token; 2.2: RoPE in the
 * numerator only):
 *   O_i = phi~(Q_i) . S / (phi(Q_i) . z + eps),  S = kv_state[b][h], z = ksum_state[b][h]
 * This is the last step of every other call, on its own: queries read a state
 * that is already complete (for example one committed by state_update).
 * q: input [B][H][N][D]; o: output, same shape and dtype, must not overlap q
 * or the states; kv_state [B][H][D][D] and ksum_state [B][H][D] are read only.
 * No workspace is used. */
int sana_linattn_apply(const void* q, void* o, const float* kv_state, const float* ksum_state,
                       int B, int H, int64_t N, int D, int dtype, float eps,
                       const sana_rope* rope, void* hip_stream);

/* The temporal convolution of block inference and its cache (the third part
 * of the block-inference cache, "SANA-Video" paper notes section 4: the conv
 * cache holds the temporal conv's last frame).  The Spatial-Temporal Mix-FFN
 * uses 3x1x1 temporal filters (news article, "Design details") entering
 * through a shortcut (paper notes, section 3 Stage 2); read as depthwise:
 *   y[b][f][s][c] = x[b][f][s][c] + w[c][0] x[b][f-1][s][c] + w[c][1] x[b][f][s][c]
 *                   + w[c][2] x[b][f+1][s][c] + bias[c]
 * x[b][-1] = cache_in[b] (zeros when cache_in is NULL: the first chunk);
 * x[b][F] = 0 (a chunk sees no later frame).  cache_out (may equal cache_in,
 * or NULL) receives x[b][F-1], the cache for the next chunk (a commit).
 * x, y: [B][F][S][C] device arrays of dtype (F frames of S spatial tokens, C
 * channels, C a multiple of 8), 16-byte aligned; y overlaps nothing.  w:
 * [C][3] fp32; bias: [C] fp32 or NULL (both 16-byte aligned); cache_in,
 * cache_out: [B][S][C] of dtype.  F = 0 or B*S*C = 0 is a no-op.  fp32 arithmetic, bf16 rounded to
 * nearest even at the store. */
int sana_linattn_temporal_conv3(const void* x, void* y, const float* w, const float* bias,
                                const void* cache_in, void* cache_out,
                                int B, int F, int64_t S, int C, int dtype, void* hip_stream);

/* Host-side builder of 3D RoPE tables ("SANA-Video" paper notes, section 3
 * Stage 2, rotary position encoding extended to space-time).  Token
 * n = (t*Hl + h)*Wl + w; the first dt dims (dt/2 pairs) turn with t, the next
 * dh with h, the last dw with w; pair k of an axis of width d_a turns by
 * coordinate * base^(-2k/d_a).  Angles are formed in double precision and
 * their cosine and sine rounded to float.  cos_host, sin_host: host arrays of
 * T*Hl*Wl*(D/2) floats, written row-major [n][p].  dt, dh, dw must be even,
 * non-negative and sum to D. */
int sana_linattn_rope3d_table(int T, int Hl, int Wl, int D, int dt, int dh, int dw, double base,
                              float* cos_host, float* sin_host);

/* Host-side builder of the per-axis form of the same 3D RoPE (see sana_rope):
 * cos_host, sin_host receive T*dt/2 + Hl*dh/2 + Wl*dw/2 floats, the t table
 * [T][dt/2], then the h table [Hl][dh/2], then the w table [Wl][dw/2]; entry
 * [x][k] of an axis of width d_a is the cosine (sine) of x * base^(-2k/d_a),
 * the same float as in sana_linattn_rope3d_table.  Use with grid = {T, Hl, Wl}
 * and pairs = {dt/2, dh/2, dw/2}. */
int sana_linattn_rope3d_axes(int T, int Hl, int Wl, int D, int dt, int dh, int dw, double base,
                             float* cos_host, float* sin_host);

/* Static string naming a status code. */
const char* sana_linattn_status_string(int status);

/* Static string: the first 16 hex digits of the SHA-256 over the kernel
 * sources the library was compiled from (every csrc *.h and *.hip file, its
 * name, a zero byte, then its bytes, in name order), as the build passes it in;
 * "unknown" for a build that did not.  A caller holding the sources can compare
 * it with their hash and refuse a library built from other sources. */
const char* sana_linattn_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* SANA_LINATTN_H */
