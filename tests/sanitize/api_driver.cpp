// Runs every entry point of the C ABI through its host-side argument checks
// (and, with valid arguments, up to the stubbed launch), so that a build with
// -fsanitize=address,undefined sees every validation path.  Prints one line
// per failed expectation and exits non-zero if there was any.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "fa.h"

extern int g_launches;
extern long long g_last_rows;

static int g_fail = 0;

#define EXPECT(expr, want)                                                              \
  do {                                                                                  \
    const int got_ = (expr);                                                            \
    if (got_ != (want)) {                                                               \
      std::printf("FAIL line %d: %s -> %d, want %d\n", __LINE__, #expr, got_, (want)); \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

// 256-byte aligned host buffers stand in for device tensors: the checks only
// look at the addresses, and the stubbed launchers never dereference them.
alignas(256) static unsigned char buf[8][4096];

int main() {
  void* P = buf[0];
  void* P2 = buf[1];
  void* W = buf[2];
  void* MIS = buf[3] + 8;                     // 8-byte aligned only
  int32_t* I = reinterpret_cast<int32_t*>(buf[4]);
  int32_t* IMIS = reinterpret_cast<int32_t*>(buf[4] + 2);
  float* F = reinterpret_cast<float*>(buf[5]);
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();

  // ---- status strings
  for (int s = 1; s >= -12; --s) {
    const char* t = fa_status_string(s);
    if (t == nullptr || std::strlen(t) == 0) { std::printf("FAIL status %d\n", s); ++g_fail; }
  }
  EXPECT(fa_version() >= 100, 1);

  // ---- fa_fwd / fa_fwd_offset
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, 64, 64, 0.125f, 1, 7, nullptr), FA_ERR_DTYPE);
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 0, 64, 64, 0.125f, 1, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P2, F, -1, 1, 64, 64, 0.125f, 1, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, 0, 64, 0.125f, 1, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, (1 << 20) + 1, 64, 0.125f, 1, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, 64, 64, nan, 1, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, 64, 64, inf, 1, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, 64, 96, 0.125f, 1, 1, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(nullptr, P, P, P2, F, 1, 1, 64, 64, 0.125f, 1, 1, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd(P, P, MIS, P2, F, 1, 1, 64, 64, 0.125f, 1, 1, nullptr), FA_ERR_ALIGN);
  // 2^31 bytes per head do not fit a buffer resource
  EXPECT(fa_fwd(P, P, P, P2, F, 1, 1, 1 << 20, 1024, 0.125f, 1, 0, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 64, 64, 0.125f, 1, 1, nullptr),
         FA_OK);
  // grid-size overflow: B * H * tiles beyond 2^31
  EXPECT(fa_fwd(P, P, P, P2, F, 1 << 20, 1 << 10, 1 << 12, 64, 0.125f, 1, 1, nullptr),
         FA_ERR_SHAPE);
  int before = g_launches;
  EXPECT(fa_fwd(P, P, P, P2, F, 2, 3, 100, 128, -0.5f, 1, 2, nullptr), FA_OK);
  EXPECT(g_launches - before, 1);
  EXPECT(g_last_rows == 600, 1);
  const long long big = 1LL << 61;
  EXPECT(fa_fwd_offset(P, P, P, P2, F, 1, 1, 64, 32, 64, big, 0, 0.1f, 1, 1, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_fwd_offset(P, P, P, P2, F, 1, 1, 64, 32, 64, -(1LL << 60), 1LL << 60, 0.1f, 1, 1,
                       nullptr),
         FA_OK);
  EXPECT(fa_fwd_offset(P, P, P, P2, F, 1, 1, 64, 0, 64, 0, 0, 0.1f, 1, 1, nullptr), FA_ERR_SHAPE);
  // ---- fa_fwd_offset_accumulate (same checks, one launch when valid)
  EXPECT(fa_fwd_offset_accumulate(P, P, P, P2, F, 1, 1, 64, 32, 64, big, 0, 0.1f, 1, 1, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_fwd_offset_accumulate(P, P, P, nullptr, F, 1, 1, 64, 32, 64, 0, 0, 0.1f, 1, 1,
                                  nullptr),
         FA_ERR_NULL);
  before = g_launches;
  EXPECT(fa_fwd_offset_accumulate(P, P, P, P2, F, 1, 2, 64, 32, 64, 100, 0, 0.1f, 1, 1, nullptr),
         FA_OK);
  EXPECT(g_launches - before, 1);

  // ---- fa_merge
  EXPECT(fa_merge(P, F, P, F, P2, F, 1, 1, 64, 64, 9, nullptr), FA_ERR_DTYPE);
  EXPECT(fa_merge(P, F, P, F, P2, F, 1, 1, 64, 80, 1, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_merge(P, nullptr, P, F, P2, F, 1, 1, 64, 64, 1, nullptr), FA_ERR_NULL);
  EXPECT(fa_merge(MIS, F, P, F, P2, F, 1, 1, 64, 64, 1, nullptr), FA_ERR_ALIGN);
  // output overlapping an input with a shift is refused; the same buffer is allowed
  EXPECT(fa_merge(buf[6], F, P, F, buf[6] + 16, F + 64, 1, 1, 8, 64, 1, nullptr), FA_ERR_INVALID);
  EXPECT(fa_merge(buf[6], F, P, F + 64, buf[6], F, 1, 1, 8, 64, 1, nullptr), FA_OK);

  // ---- fa_bwd
  const size_t ws = fa_bwd_workspace_size(2, 3, 100, 128);
  EXPECT(ws >= 2 * 2 * 3 * 100 * sizeof(float), 1);
  EXPECT(fa_bwd_workspace_size(0, 3, 100, 128) == 0, 1);
  float* g = F;
  EXPECT(fa_bwd(P, P, P, P, P, F, g, g, g, 2, 3, 100, 128, 0.1f, 1, 1, W, ws, nullptr), FA_OK);
  EXPECT(fa_bwd(P, P, P, P, P, F, g, g, g, 2, 3, 100, 128, 0.1f, 1, 1, W, ws - 1, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(P, P, P, P, P, F, g, g, g, 2, 3, 100, 128, 0.1f, 1, 1, nullptr, ws, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(P, P, P, P, P, F, g, g, g, 2, 3, 100, 128, 0.1f, 1, 0, W, ws, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_bwd(P, P, P, P, nullptr, F, g, g, g, 2, 3, 100, 128, 0.1f, 1, 1, W, ws, nullptr),
         FA_ERR_NULL);
  EXPECT(fa_bwd(P, P, P, P, P, F, g, g, g, 2, 3, 100, 128, nan, 1, 1, W, ws, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_bwd(P, P, P, MIS, P, F, g, g, g, 2, 3, 100, 128, 0.1f, 1, 1, W, ws, nullptr),
         FA_ERR_ALIGN);
  EXPECT(fa_bwd(P, P, P, P, P, F, g, g, g, 1 << 12, 1 << 12, 128 * 128, 128, 0.1f, 1, 1, W, ws,
                nullptr),
         FA_ERR_SHAPE);   // 2^31 workgroups per kernel

  // ---- decode (workspace and static-scratch entry points)
  const size_t dws = fa_paged_decode_workspace_size(64, 32, 128, 256, 16);
  EXPECT(dws > 0, 1);
  EXPECT(fa_paged_decode_workspace_size(0, 32, 128, 256, 16) == 0, 1);
  EXPECT(fa_paged_decode(P, P, P, I, I, 16, 64, 32, 128, 256, 9000, 0.088f, P2, F, 1, W, dws,
                         nullptr),
         FA_OK);
  EXPECT(fa_paged_decode(P, P, P, I, I, 16, 64, 32, 128, 256, 9000, 0.088f, P2, F, 1, W, dws - 1,
                         nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_paged_decode(P, P, P, I, I, 8, 64, 32, 128, 256, 9000, 0.088f, P2, F, 1, W, dws,
                         nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_paged_decode(P, P, P, I, I, 16, 64, 32, 96, 256, 9000, 0.088f, P2, F, 1, W, dws,
                         nullptr),
         FA_ERR_UNSUPPORTED);
  // any head count (here 30) and head dim 64 are accepted
  EXPECT(fa_paged_decode(P, P, P, I, I, 16, 64, 30, 64, 256, 9000, 0.088f, P2, F, 1, W, dws,
                         nullptr),
         FA_OK);
  EXPECT(fa_paged_decode(P, P, P, IMIS, I, 16, 64, 32, 128, 256, 9000, 0.088f, P2, F, 1, W, dws,
                         nullptr),
         FA_ERR_ALIGN);
  EXPECT(fa_paged_decode_gqa(P, P, P, I, I, 16, 64, 32, 5, 128, 256, 9000, 0.088f, P2, F, 1, W,
                             dws, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_paged_decode_gqa(P, P, P, I, I, 16, 1 << 25, 32, 8, 128, 256, 9000, 0.088f, P2, F, 1,
                             W, dws, nullptr),
         FA_ERR_SHAPE);   // num_seqs * H >= 2^30
  EXPECT(fa_paged_decode_gqa(P, P, P, I, I, 16, 64, 32, 8, 128, 256, 9000, 0.088f, P2, F, 1, W,
                             dws, nullptr),
         FA_OK);
  EXPECT(fa_paged_decode_gqa_noalloc(P, P, P, I, I, 16, 64, 32, 8, 128, 256, 9000, 0.088f, P2, F,
                                     1, nullptr),
         FA_OK);
  EXPECT(fa_paged_decode_gqa_noalloc(P, P, P, I, I, 16, 4000, 32, 8, 128, 256, 9000, 0.088f, P2,
                                     F, 1, nullptr),
         FA_ERR_SCRATCH);
  EXPECT(fa_paged_decode_gqa_noalloc(nullptr, P, P, I, I, 16, 64, 32, 8, 128, 256, 9000, 0.088f,
                                     P2, F, 1, nullptr),
         FA_ERR_NULL);
  EXPECT(fa_paged_decode_gqa_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, 16, 0, 32, 8,
                                     128, 256, 9000, 0.088f, nullptr, nullptr, 1, nullptr),
         FA_OK);

  // ---- prefill
  EXPECT(fa_paged_prefill(P, I, P, P, I, I, 8, 8192, 32, 8, 128, 16, 256, 9000, 1024, 0.088f, 1, P2,
                          F, 1, nullptr),
         FA_OK);
  EXPECT(fa_paged_prefill(P, I, P, P, I, I, 8, 8192, 32, 7, 128, 16, 256, 9000, 1024, 0.088f, 1, P2,
                          F, 1, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_paged_prefill(P, I, P, P, I, I, 8, 8192, 32, 8, 96, 16, 256, 9000, 1024, 0.088f, 1, P2,
                          F, 1, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_paged_prefill(P, I, P, P, I, I, 8, 1 << 24, 32, 8, 128, 16, 256, 9000, 1024, 0.088f, 1,
                          P2, F, 1, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_paged_prefill(P, IMIS, P, P, I, I, 8, 8192, 32, 8, 128, 16, 256, 9000, 1024, 0.088f, 1,
                          P2, F, 1, nullptr),
         FA_ERR_ALIGN);
  EXPECT(fa_paged_prefill(P, I, P, P, I, I, 0, 8192, 32, 8, 128, 16, 256, 9000, 1024, 0.088f, 1, P2,
                          F, 1, nullptr),
         FA_OK);

  // ---- append
  const size_t aws = fa_paged_kv_append_workspace_size(64);
  EXPECT(aws >= 64 * sizeof(int32_t), 1);
  EXPECT(fa_paged_kv_append(P, P, P, P, I, I, I, I, I, 64, 8, 128, 16, 256, 9000, 100, 1, W, aws,
                            nullptr),
         FA_OK);
  EXPECT(fa_paged_kv_append(P, P, P, P, I, I, I, I, I, 64, 8, 128, 16, 256, 9000, 100, 1, W,
                            aws - 1, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_paged_kv_append(P, P, P, P, I, I, nullptr, I, I, 64, 8, 128, 16, 256, 9000, 100, 1, W,
                            aws, nullptr),
         FA_ERR_NULL);
  EXPECT(fa_paged_kv_append(P, P, P, P, I, I, nullptr, I, I, 64, 8, 128, 16, 256, 9000, 0, 1, W,
                            aws, nullptr),
         FA_OK);
  EXPECT(fa_paged_kv_append(P, P, P, P, I, I, I, I, I, 64, 3, 2, 16, 256, 9000, 100, 1, W, aws,
                            nullptr),
         FA_ERR_UNSUPPORTED);

  std::printf("%s: %d failed expectations, %d stubbed launches\n", g_fail ? "FAIL" : "OK", g_fail,
              g_launches);
  return g_fail ? 1 : 0;
}
