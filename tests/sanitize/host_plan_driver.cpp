// host_plan_driver.cpp -- exercises the host-side validation and slot / size
// arithmetic of the library (host_plan.cpp) on valid and invalid batch
// descriptions, built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py.  Pure host code: no HIP call is made.  Exits 0
// when every status is the documented one; any sanitizer report aborts.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "host_plan.h"

using namespace flare;

static int g_bad = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_bad;                                                           \
    }                                                                    \
  } while (0)

static flare_varlen make(const std::vector<int32_t> &cu, const std::vector<int32_t> &pl, bool dev = true) {
  static int32_t dummy[1];
  flare_varlen v{};
  v.num_docs = (int32_t)pl.size();
  v.cu_seqlens_host = cu.data();
  v.prompt_lens_host = pl.data();
  v.cu_seqlens = dev ? dummy : nullptr;
  v.prompt_lens = dev ? dummy : nullptr;
  return v;
}

int main() {
  // ---- packed-batch validation
  {
    std::vector<int32_t> cu{0, 100, 100, 164, 171}, pl{16, 0, 32, 4};
    flare_varlen v = make(cu, pl);
    VarlenInfo vi;
    EXPECT(check_varlen(&v, 4, &vi) == FLARE_OK);
    EXPECT(vi.total_tokens == 171 && vi.max_len == 100 && vi.total_chunks == 4 + 0 + 2 + 1);
    EXPECT(check_varlen(&v, 8, &vi) == FLARE_ERR_ALIGN);  // prompt 4 is not a multiple of 8
    EXPECT(check_varlen(nullptr, 4, &vi) == FLARE_ERR_NULL);
    EXPECT(check_varlen(&v, 0, &vi) == FLARE_ERR_SHAPE);
    flare_varlen nd = make(cu, pl, false);
    EXPECT(check_varlen(&nd, 4, &vi) == FLARE_ERR_NULL);
  }
  {
    std::vector<int32_t> cu{1, 10}, pl{0};
    flare_varlen v = make(cu, pl);
    EXPECT(check_varlen(&v, 1, nullptr) == FLARE_ERR_SHAPE);  // cu[0] != 0
  }
  {
    std::vector<int32_t> cu{0, 10, 5}, pl{0, 0};
    flare_varlen v = make(cu, pl);
    EXPECT(check_varlen(&v, 1, nullptr) == FLARE_ERR_SHAPE);  // decreasing
  }
  {
    std::vector<int32_t> cu{0, 10}, pl{12};
    flare_varlen v = make(cu, pl);
    EXPECT(check_varlen(&v, 4, nullptr) == FLARE_ERR_SHAPE);  // prompt longer than the document
  }
  {
    std::vector<int32_t> cu{0}, pl{0};
    flare_varlen v = make(cu, pl, false);
    v.num_docs = 0;  // no documents: host arrays still given, device arrays may be NULL
    VarlenInfo vi;
    EXPECT(check_varlen(&v, 4, &vi) == FLARE_OK && vi.total_tokens == 0);
  }
  // ---- shapes
  {
    flare_gdn_shape s{16, 128, 128, 4, FLARE_BF16, 0, 0.f};
    EXPECT(check_gdn_shape(&s) == FLARE_OK);
    EXPECT(resolve_scale(&s) > 0.0883f && resolve_scale(&s) < 0.0884f);
    flare_gdn_shape t = s; t.d_v = 64;
    EXPECT(check_gdn_shape(&t) == FLARE_ERR_UNSUPPORTED);
    t = s; t.block_size = 3;
    EXPECT(check_gdn_shape(&t) == FLARE_ERR_UNSUPPORTED);
    t = s; t.block_size = 64;
    EXPECT(check_gdn_shape(&t) == FLARE_ERR_UNSUPPORTED);
    t = s; t.flags = 8;
    EXPECT(check_gdn_shape(&t) == FLARE_ERR_UNSUPPORTED);
    t = s; t.num_heads = 0;
    EXPECT(check_gdn_shape(&t) == FLARE_ERR_SHAPE);
    EXPECT(check_gdn_shape(nullptr) == FLARE_ERR_NULL);
  }
  // ---- checkpoint slots: distinct per (document, chunk), inside the slot count
  {
    std::vector<int32_t> cu{0, 31, 95, 95, 160, 1000}, pl{0, 0, 0, 0, 0};
    flare_varlen v = make(cu, pl);
    VarlenInfo vi;
    EXPECT(check_varlen(&v, 1, &vi) == FLARE_OK);
    for (int stride = 1; stride <= 4; ++stride) {
      const int64_t nslots = ckpt_num_slots(vi, stride);
      std::vector<int> seen((size_t)nslots, 0);
      for (int i = 0; i < v.num_docs; ++i) {
        const int n = cu[i + 1] - cu[i];
        for (int c = 0; c * kChunk < n; c += stride) {
          const int64_t s = ckpt_slot(cu[i], i, c, stride);
          EXPECT(s >= 0 && s < nslots);
          if (s >= 0 && s < nslots) {
            EXPECT(seen[(size_t)s] == 0);
            seen[(size_t)s] = 1;
          }
        }
      }
    }
    flare_gdn_shape s{2, 128, 128, 4, FLARE_BF16, 0, 0.f};
    EXPECT(bwd_workspace_bytes(vi, &s) > fwd_workspace_bytes(vi, &s) / 2);
    EXPECT(fwd_uses_chunk_matrices(&s) && bwd_uses_scan_pack(&s));
  }
  // ---- serving slots
  {
    const int32_t ok[3] = {4, 0, 2}, dup[3] = {4, 0, 4}, out[2] = {1, 5};
    EXPECT(check_slots_host(3, ok, 5) == FLARE_OK);
    EXPECT(check_slots_host(3, dup, 5) == FLARE_ERR_SHAPE);
    EXPECT(check_slots_host(2, out, 5) == FLARE_ERR_SHAPE);
    EXPECT(check_slots_host(3, nullptr, 5) == FLARE_OK);
    flare_gdn_shape s{2, 128, 128, 4, FLARE_BF16, 0, 0.f};
    float pool[1];
    int32_t dslot[1];
    EXPECT(check_block_step(3, dslot, ok, pool, 5, &s, pool, pool, pool, pool, pool, pool, FLARE_BLOCK_EVAL) ==
           FLARE_OK);
    EXPECT(check_block_step(3, dslot, ok, pool, 5, &s, pool, pool, pool, pool, pool, nullptr, FLARE_BLOCK_EVAL) ==
           FLARE_ERR_NULL);
    EXPECT(check_block_step(6, dslot, nullptr, pool, 5, &s, pool, pool, pool, pool, pool, pool, FLARE_BLOCK_COMMIT) ==
           FLARE_ERR_SHAPE);
    EXPECT(check_block_step(3, dslot, ok, pool, 5, &s, pool, pool, pool, pool, pool, pool, 7) == FLARE_ERR_SHAPE);
  }
  // ---- Route I counts
  {
    std::vector<int32_t> cu{0, 100, 100, 164}, pl{16, 0, 32};
    flare_varlen v = make(cu, pl);
    EXPECT(route1_num_blocks(&v, 4) == (84 + 3) / 4 + 0 + 8);
    EXPECT(route1_num_windows(&v) == (4 - 0) + 0 + (2 - 1));
  }
  // ---- ShortConv and the QKV prologue
  {
    std::vector<int32_t> cu{0, 300, 600}, pl{0, 0};
    flare_varlen v = make(cu, pl);
    VarlenInfo vi;
    int x[1];
    float w[1];
    EXPECT(check_shortconv(&v, 4, 96, 4, FLARE_BF16, x, x, w, 0, x, x, &vi) == FLARE_OK);
    EXPECT(check_shortconv(&v, 4, 12, 4, FLARE_BF16, x, x, w, 0, x, x, &vi) == FLARE_ERR_ALIGN);
    EXPECT(check_shortconv(&v, 4, 96, 9, FLARE_BF16, x, x, w, 0, x, x, &vi) == FLARE_ERR_UNSUPPORTED);
    EXPECT(check_shortconv(&v, 4, 96, 4, FLARE_BF16, x, x, w, 2, x, x, &vi) == FLARE_ERR_UNSUPPORTED);
    EXPECT(check_shortconv(&v, 4, 96, 4, FLARE_BF16, nullptr, x, w, 0, x, x, &vi) == FLARE_ERR_NULL);
    EXPECT(shortconv_bwd_workspace_bytes(vi, 96, 4, 3) == (size_t)3 * 3 * 96 * 5 * 4 + 256);
    const void *xs[3] = {x, x, x};
    const float *ws[3] = {w, w, w};
    EXPECT(check_qkv_prologue(&v, 4, 4, 32, 4, FLARE_BF16, xs, xs, ws, 0, 1, xs, xs, &vi) == FLARE_OK);
    EXPECT(check_qkv_prologue(&v, 4, 4, 24, 4, FLARE_BF16, xs, xs, ws, 0, 1, xs, xs, &vi) == FLARE_ERR_UNSUPPORTED);
  }
  // ---- error messages stay inside their buffer
  {
    char big[2048];
    for (int i = 0; i < 2047; ++i) big[i] = 'x';
    big[2047] = '\0';
    fail(FLARE_ERR_SHAPE, "%s", big);
    EXPECT(last_error()[0] == 'x');
    clear_error();
    EXPECT(last_error()[0] == '\0');
  }
  if (g_bad) {
    std::fprintf(stderr, "%d checks failed\n", g_bad);
    return 1;
  }
  std::printf("host_plan checks passed\n");
  return 0;
}
