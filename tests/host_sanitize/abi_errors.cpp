// Host-only driver of the C ABI's argument checks, built and run under
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitize.py).
// Every compute call below carries an argument error, so the library must
// return its status before touching the (fake) device pointers or the GPU; the
// host-side RoPE table builders and workspace-size functions run for real on
// host memory.  Exit status 0 when every call returns what the header states.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "sana_linattn.h"

static int failures = 0;

#define EXPECT(call, want)                                                                          \
  do {                                                                                              \
    const long long got_ = (long long)(call);                                                       \
    if (got_ != (long long)(want)) {                                                                \
      std::fprintf(stderr, "%s:%d: %s -> %lld, want %lld\n", __FILE__, __LINE__, #call, got_,     \
                   (long long)(want));                                                              \
      ++failures;                                                                                   \
    }                                                                                               \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }

int main() {
  const int BF = SANA_DT_BF16, F32 = SANA_DT_F32;
  void *q = P(0x10000000), *k = P(0x20000000), *v = P(0x30000000), *o = P(0x40000000), *ws = P(0x50000000);
  float *S = F(0x60000000), *Z = F(0x61000000);
  const size_t nws = sana_linattn_workspace_bytes(1, 2, 640, 32, BF, 0);
  const size_t nws_rope = sana_linattn_workspace_bytes(1, 2, 640, 32, BF, 1);

  // workspace sizes: pure host functions over a range of sizes, invalid ones 0
  EXPECT(sana_linattn_workspace_bytes(0, 2, 10, 32, BF, 0), 0);
  EXPECT(sana_linattn_workspace_bytes(1, 2, 10, 64, BF, 0), 0);
  EXPECT(sana_linattn_workspace_bytes(1, 2, -1, 32, BF, 0), 0);
  EXPECT(sana_linattn_workspace_bytes(1, 2, 10, 32, 9, 0), 0);
  EXPECT(sana_linattn_forward_launches(0, 2, 10, 10, 32, BF, 0, 1), 0);
  EXPECT(sana_linattn_forward_launches(1, 2, 10, 0, 32, BF, 0, 1), 0);
  EXPECT(sana_linattn_forward_launches(1, 2, 10, 10, 32, BF, 5, 1), 0);
  EXPECT(sana_linattn_forward_launches(1, 2, -3, 10, 32, BF, 0, 1), 0);
  EXPECT(sana_linattn_forward_launches(4, 36, 1024, 1024, 32, BF, 0, 1), 1);
  for (int B = 1; B <= 3; ++B)
    for (int H = 1; H <= 80; H += 13)
      for (int64_t N : {1LL, 63LL, 1024LL, 4680LL, 16384LL, 1000003LL}) {
        const size_t a = sana_linattn_workspace_bytes(B, H, N, 32, BF, 0);
        if (a == 0 || a % 256 != 0) {
          std::fprintf(stderr, "workspace_bytes(%d, %d, %lld) = %zu\n", B, H, (long long)N, a);
          ++failures;
        }
        for (int64_t chunk : {1LL, 7LL, 4680LL})
          if (sana_linattn_block_causal_workspace_bytes(B, H, N, chunk, 32, BF, 1) == 0) ++failures;
        (void)sana_linattn_project_state_workspace_bytes(B, H, N, 2240, 32, BF);
        for (int form = 0; form <= 2; ++form) {
          const int n = sana_linattn_forward_launches(B, H, N, N, 32, BF, form, 1);
          if (n < 1 || n > 3) ++failures;
          if (sana_linattn_forward_launches(B, H, N, 1000, 32, BF, form, 0) < 2) ++failures;
        }
      }
  EXPECT(sana_linattn_block_causal_workspace_bytes(1, 2, 100, 0, 32, BF, 0), 0);
  EXPECT(sana_linattn_backward_workspace_bytes(1, 2, 100, -3, 32, BF, 0), 0);
  EXPECT(sana_linattn_project_state_workspace_bytes(1, 2, 100, 48, 32, BF), 0);

  // forward
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 48, BF, 1e-6f, nullptr, ws, nws, nullptr), SANA_ERR_UNSUPPORTED);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, 7, 1e-6f, nullptr, ws, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, o, -1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, -1.f, nullptr, ws, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, NAN, nullptr, ws, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(nullptr, k, v, o, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, P(0x40000008), 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, q, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws - 1, nullptr),
         SANA_ERR_WORKSPACE);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, nullptr, nullptr, nws, nullptr),
         SANA_ERR_WORKSPACE);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, nullptr, P(0x50000040), nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, nullptr, q, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, (int64_t)1 << 62, 32, BF, 1e-6f, nullptr, ws, nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward(nullptr, nullptr, nullptr, nullptr, 1, 2, 0, 32, BF, 1e-6f, nullptr, nullptr, 0,
                              nullptr),
         SANA_OK);

  // RoPE argument checks (full tables and per-axis form)
  sana_rope r{};
  r.cos = F(0x70000000);
  r.sin = F(0x71000000);
  r.n_pos = 639;
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);
  r.n_pos = 700;
  r.pos_offset = 61;
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);
  r.pos_offset = 0;
  r.pairs[0] = 4;  // pairs without a grid
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);
  r.n_pos = 640;
  r.grid[0] = 4; r.grid[1] = 8; r.grid[2] = 20;
  r.pairs[0] = 3; r.pairs[1] = 6; r.pairs[2] = 7;  // odd pair count
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);
  r.pairs[0] = 4; r.pairs[1] = 6; r.pairs[2] = 5;  // 15 pairs
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);
  r.pairs[2] = 6;
  r.grid[2] = 21;  // grid does not match n_pos
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);
  r.grid[2] = 20;
  r.cos = F(0x50000100);  // a table inside the workspace
  EXPECT(sana_linattn_forward(q, k, v, o, 1, 2, 640, 32, BF, 1e-6f, &r, ws, nws_rope, nullptr), SANA_ERR_INVALID);

  // strided views
  sana_layout bad{-1, 32, 32}, tiny{0, 32, 16}, mis{0, 32, 40}, overlapping{0, 16, 32};
  EXPECT(sana_linattn_forward_strided(q, k, v, o, &bad, nullptr, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws,
                                      nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward_strided(q, k, v, o, &tiny, nullptr, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws,
                                      nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward_strided(q, k, v, o, nullptr, &mis, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws,
                                      nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_forward_strided(q, k, v, o, nullptr, &overlapping, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws,
                                      nullptr),
         SANA_ERR_INVALID);

  // state_update, apply, block_forward (and its allocation-free form), block_causal
  EXPECT(sana_linattn_state_update(k, v, nullptr, Z, 1, 2, 640, 32, BF, nullptr, ws, nws, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_state_update(k, v, S, F(0x60000000 + 1024), 1, 2, 640, 32, BF, nullptr, ws, nws, nullptr),
         SANA_ERR_INVALID);  // the key sum inside the state (2 heads x 4 KiB)
  EXPECT(sana_linattn_apply(q, o, S, Z, 1, 2, 640, 32, BF, -2.f, nullptr, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_apply(q, q, S, Z, 1, 2, 640, 32, BF, 1e-6f, nullptr, nullptr), SANA_ERR_INVALID);
  EXPECT(sana_linattn_block_forward(q, k, v, o, S, nullptr, nullptr, nullptr, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws,
                                    nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_block_forward(q, k, v, o, S, Z, S + 8, Z, 1, 2, 640, 32, BF, 1e-6f, nullptr, ws, nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_block_forward_noalloc(q, k, v, o, nullptr, nullptr, nullptr, nullptr, 1, 4000, 64, 32, BF,
                                            1e-6f, nullptr, nullptr),
         SANA_ERR_WORKSPACE);
  EXPECT(sana_linattn_block_causal(q, k, v, o, nullptr, nullptr, S, Z, 1, 2, 640, 0, 32, BF, 1e-6f, nullptr, ws,
                                   nws, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_block_causal(q, k, v, o, nullptr, nullptr, S, Z, 1, 2, 640, 64, 32, BF, 1e-6f, nullptr, ws,
                                   nws, nullptr),
         SANA_ERR_WORKSPACE);  // ten chunks need more than one chunk's workspace

  // backward family
  void *dq = P(0x80000000), *dk = P(0x81000000), *dv = P(0x82000000), *dout = P(0x83000000);
  const size_t nbw = sana_linattn_backward_workspace_bytes(1, 2, 640, 64, 32, BF, 0);
  EXPECT(sana_linattn_backward(q, k, v, dout, dq, dk, dv, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 2,
                               640, 0, 32, BF, 1e-6f, nullptr, ws, nbw, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_backward(q, k, v, dout, q, dk, dv, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 2,
                               640, 64, 32, BF, 1e-6f, nullptr, ws, nbw, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_backward(q, k, v, dout, dq, dk, dv, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 2,
                               640, 64, 32, BF, 1e-6f, nullptr, ws, nbw - 256, nullptr),
         SANA_ERR_WORKSPACE);
  EXPECT(sana_linattn_backward_strided(q, k, v, dout, dq, dk, dv, &bad, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, 1, 2, 640, 64, 32, BF, 1e-6f, nullptr, ws, nbw, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_backward_saved(q, k, v, dout, dq, dk, dv, nullptr, nullptr, S, nullptr, nullptr, nullptr, 1, 2,
                                     640, 64, 32, BF, 1e-6f, nullptr, ws, nbw, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_state_update_backward(k, v, S, Z, k, dv, 1, 2, 640, 32, BF, nullptr, nullptr),
         SANA_ERR_INVALID);

  // fused projections
  const size_t nps = sana_linattn_project_state_workspace_bytes(1, 2, 1000, 64, 32, BF);
  EXPECT(sana_linattn_project_state(q, k, v, S, Z, 1, 2, 1000, 48, 32, BF, nullptr, ws, nps, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_project_state(q, k, v, S, Z, 1, 2, 1000, 64, 32, F32, nullptr, ws, nps, nullptr),
         SANA_ERR_UNSUPPORTED);
  EXPECT(sana_linattn_project_state(q, k, v, S, Z, 1, 2, 1000, 64, 32, BF, nullptr, ws, nps - 1, nullptr),
         SANA_ERR_WORKSPACE);
  EXPECT(sana_linattn_project_apply(q, k, o, nullptr, S, Z, 1, 2, 1000, 64, 32, BF, -1.f, nullptr, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_project_apply(q, k, q, nullptr, S, Z, 1, 2, 1000, 64, 32, BF, 1e-6f, nullptr, nullptr),
         SANA_ERR_INVALID);

  // temporal conv
  EXPECT(sana_linattn_temporal_conv3(q, o, S, nullptr, nullptr, nullptr, 1, 3, 100, 12, BF, nullptr),
         SANA_ERR_INVALID);
  EXPECT(sana_linattn_temporal_conv3(q, q, S, nullptr, nullptr, nullptr, 1, 3, 100, 16, BF, nullptr),
         SANA_ERR_INVALID);

  // host RoPE builders, for real: every entry written, in range, and the
  // per-axis tables' entries equal the full tables' for the same angles
  const int T = 3, Hl = 5, Wl = 7, n = T * Hl * Wl;
  std::vector<float> c(n * 16), s(n * 16);
  EXPECT(sana_linattn_rope3d_table(T, Hl, Wl, 32, 8, 12, 12, 10000.0, c.data(), s.data()), SANA_OK);
  std::vector<float> ca(T * 4 + Hl * 6 + Wl * 6), sa(ca.size());
  EXPECT(sana_linattn_rope3d_axes(T, Hl, Wl, 32, 8, 12, 12, 10000.0, ca.data(), sa.data()), SANA_OK);
  for (int i = 0; i < n * 16; ++i)
    if (!(std::fabs(c[i] * c[i] + s[i] * s[i] - 1.f) < 1e-5f)) ++failures;
  for (int t = 0; t < T; ++t)
    for (int p = 0; p < 4; ++p)
      if (ca[t * 4 + p] != c[(t * Hl * Wl) * 16 + p]) ++failures;
  EXPECT(sana_linattn_rope3d_table(T, Hl, Wl, 32, 8, 12, 11, 10000.0, c.data(), s.data()), SANA_ERR_INVALID);
  EXPECT(sana_linattn_rope3d_table(T, Hl, Wl, 32, 8, 12, 12, -1.0, c.data(), s.data()), SANA_ERR_INVALID);
  EXPECT(sana_linattn_rope3d_axes(T, Hl, Wl, 32, 8, 12, 12, 10000.0, nullptr, sa.data()), SANA_ERR_INVALID);

  for (int code = -6; code <= 2; ++code)
    if (!sana_linattn_status_string(code) || !std::strlen(sana_linattn_status_string(code))) ++failures;

  if (failures) std::fprintf(stderr, "%d check(s) failed\n", failures);
  else std::printf("all ABI error paths behaved\n");
  return failures ? 1 : 0;
}
