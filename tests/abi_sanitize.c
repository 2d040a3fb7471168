/* Host-side driver of the C ABI for the sanitizer build: every entry point's
 * argument checks and workspace sizing, run on the CPU under AddressSanitizer
 * and UndefinedBehaviorSanitizer.  Device pointers are stand-ins that the
 * host code never dereferences; calls whose arguments pass every check stop
 * at the device query when no GPU is present (MUSE_ERR_HIP).  Prints OK and
 * exits 0 when every expectation holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "muse_attn.h"

static int fails = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, muse_last_error()); \
      fails++;                                                         \
    }                                                                  \
  } while (0)

static void* const FAKE = (void*)0x1000;   /* 16-byte aligned stand-in */
static void* const ODD = (void*)0x1002;    /* misaligned stand-in */

static muse_attn_params glimmer_local(void) {
  muse_attn_params p = {32, 2, 128, 2048, 10000.f, 3.87f, 1e-5f, 0, 1e-6f};
  return p;
}
static muse_attn_params spark_global(void) {
  muse_attn_params p = {128, 16, 64, 0, 0.f, 5.473f, 1e-5f, 1, 1e-6f};
  return p;
}
static muse_kv_cache ring(int cap) {
  muse_kv_cache c;
  memset(&c, 0, sizeof c);
  c.kind = MUSE_KV_RING;
  c.capacity = cap;
  c.k = FAKE;
  c.v = FAKE;
  return c;
}
static muse_kv_cache paged(int max_pages, int page_tokens, int64_t num_pages) {
  muse_kv_cache c;
  memset(&c, 0, sizeof c);
  c.kind = MUSE_KV_PAGED;
  c.k = FAKE;
  c.v = FAKE;
  c.block_table = (const int32_t*)FAKE;
  c.max_pages_per_seq = max_pages;
  c.page_tokens = page_tokens;
  c.num_pages = num_pages;
  return c;
}
/* a call that passed every check stops at the device */
static int reached_device(int32_t rc) { return rc == MUSE_OK || rc == MUSE_ERR_HIP || rc == MUSE_ERR_UNSUPPORTED; }

static void workspace_sizes(void) {
  const muse_attn_params ps[2] = {glimmer_local(), spark_global()};
  for (int i = 0; i < 2; ++i) {
    const muse_attn_params* p = &ps[i];
    for (int B = 0; B <= 16; B += 4)
      for (int T = 1; T <= 262144; T *= 8) {
        const size_t a = muse_attn_prefill_workspace_size(p, B, T);
        EXPECT(B == 0 || a > 0);
        for (int ms = 0; ms <= (1 << 20); ms = ms ? ms * 16 : 1) {
          const size_t c = muse_attn_prefill_chunk_workspace_size(p, B, T, ms);
          const size_t d = muse_attn_draft_block_workspace_size(p, B, T, ms);
          EXPECT(B == 0 || c > 0);
          EXPECT(B == 0 || d > 0);
        }
      }
    muse_kv_cache r = ring(p->sliding_window > 0 ? p->sliding_window : 2048);
    muse_kv_cache g = paged(32768, 32, 1 << 20);
    for (int B = 1; B <= 64; B *= 2) {
      EXPECT(muse_attn_decode_workspace_size(p, B, 1 << 20, &g) > 0);
      if (p->sliding_window > 0) EXPECT(muse_attn_decode_workspace_size(p, B, 1 << 20, &r) > 0);
    }
  }
  /* invalid parameters size to 0 */
  muse_attn_params bad = glimmer_local();
  bad.head_dim = 96;
  EXPECT(muse_attn_prefill_workspace_size(&bad, 1, 16) == 0);
  EXPECT(muse_attn_prefill_workspace_size(NULL, 1, 16) == 0);
  EXPECT(muse_attn_draft_block_workspace_size(&bad, 1, 16, 64) == 0);
}

static void prefill_checks(void) {
  const muse_attn_params p = glimmer_local();
  const size_t ws = muse_attn_prefill_workspace_size(&p, 2, 256);
  int64_t strides[10] = {0};
  EXPECT(muse_attn_prefill(NULL, 2, 256, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws, NULL) != MUSE_OK);
  EXPECT(muse_attn_prefill(&p, -1, 256, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_INVALID_ARG);
  EXPECT(muse_attn_prefill(&p, 2, 256, NULL, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_INVALID_ARG);
  EXPECT(muse_attn_prefill(&p, 2, 256, ODD, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_INVALID_ARG);
  EXPECT(muse_attn_prefill(&p, 2, 256, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws - 1, NULL) ==
         MUSE_ERR_WORKSPACE);
  EXPECT(muse_attn_prefill(&p, 2, 256, FAKE, FAKE, FAKE, FAKE, strides, NULL, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_INVALID_ARG);   /* token strides smaller than H * D */
  EXPECT(muse_attn_prefill(&p, 0, 256, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws, NULL) == MUSE_OK);
  EXPECT(strlen(muse_last_error()) == 0);
  EXPECT(reached_device(muse_attn_prefill(&p, 2, 256, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, ws, NULL)));
  EXPECT(muse_rope_qknorm(NULL, 16, FAKE, 0, FAKE, 0, NULL, FAKE, FAKE, 0, NULL) != MUSE_OK);
  EXPECT(muse_rope_qknorm(&p, 16, FAKE, 32 * 128, FAKE, 2 * 128, NULL, FAKE, FAKE, 7, NULL) ==
         MUSE_ERR_INVALID_ARG);   /* unknown output dtype */
  EXPECT(muse_rope_qknorm(&p, 16, FAKE, 32 * 128 - 1, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
         MUSE_ERR_INVALID_ARG);   /* q token stride below Hq * D */
  EXPECT(muse_rope_qknorm(&p, 16, FAKE, 32 * 128, FAKE, 2 * 128, NULL, NULL, FAKE, 0, NULL) ==
         MUSE_ERR_INVALID_ARG);   /* q without q_out */
  EXPECT(reached_device(muse_rope_qknorm(&p, 16, FAKE, 32 * 128, FAKE, 2 * 128, NULL, FAKE, FAKE, 0, NULL)));
}

static void chunk_and_draft_checks(void) {
  const muse_attn_params p = glimmer_local();
  muse_kv_cache r = ring(2048);
  muse_kv_cache r_bad = ring(1024);
  for (int draft = 0; draft < 2; ++draft) {
    const size_t ws = draft ? muse_attn_draft_block_workspace_size(&p, 2, 16, 4096)
                            : muse_attn_prefill_chunk_workspace_size(&p, 2, 16, 4096);
    int32_t (*f)(const muse_attn_params*, int32_t, int32_t, const void*, const void*, const void*, const void*,
                 const int64_t*, const int32_t*, int32_t, const muse_kv_cache*, void*, void*, size_t, void*) =
        draft ? muse_attn_draft_block : muse_attn_prefill_chunk;
    EXPECT(f(&p, 2, -1, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 4096, &r, FAKE, FAKE, ws, NULL) == MUSE_ERR_INVALID_ARG);
    EXPECT(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, -1, &r, FAKE, FAKE, ws, NULL) == MUSE_ERR_INVALID_ARG);
    EXPECT(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 0x7FFFFFFF, &r, FAKE, FAKE, ws, NULL) ==
           MUSE_ERR_UNSUPPORTED);
    EXPECT(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 4096, NULL, FAKE, FAKE, ws, NULL) ==
           MUSE_ERR_INVALID_ARG);
    EXPECT(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 4096, &r, FAKE, FAKE, ws, NULL) == MUSE_ERR_INVALID_ARG);
    EXPECT(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 4096, &r_bad, FAKE, FAKE, ws, NULL) ==
           MUSE_ERR_INVALID_ARG);
    EXPECT(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 4096, &r, FAKE, FAKE, ws - 1, NULL) ==
           MUSE_ERR_WORKSPACE);
    EXPECT(reached_device(f(&p, 2, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 4096, &r, FAKE, FAKE, ws, NULL)));
  }
  /* the few-token drafter path: 16 tokens x 4 heads per KV head */
  muse_attn_params a = glimmer_local();
  a.num_kv_heads = 8;
  const size_t wsa = muse_attn_draft_block_workspace_size(&a, 16, 16, 131072);
  EXPECT(wsa > 0);
  EXPECT(muse_attn_draft_block(&a, 16, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 131072, &r, FAKE, FAKE, wsa - 1,
                               NULL) == MUSE_ERR_WORKSPACE);
  EXPECT(reached_device(
      muse_attn_draft_block(&a, 16, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 131072, &r, FAKE, FAKE, wsa, NULL)));
}

static void decode_checks(void) {
  const muse_attn_params p = spark_global();
  muse_kv_cache g = paged(32768, 32, 1 << 20);
  muse_kv_cache g_bad = paged(32768, 24, 1 << 20);   /* pages not a multiple of 16 */
  const size_t ws = muse_attn_decode_workspace_size(&p, 16, 1 << 20, &g);
  EXPECT(muse_attn_decode(&p, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, &g, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_INVALID_ARG);
  EXPECT(muse_attn_decode(&p, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, &g_bad, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_UNSUPPORTED);
  EXPECT(muse_attn_decode(&p, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, &g, FAKE, FAKE, ws - 1, NULL) ==
         MUSE_ERR_WORKSPACE);
  EXPECT(muse_attn_decode(&p, 16, FAKE, FAKE, FAKE, FAKE, FAKE, (1 << 20) + 1, &g, FAKE, FAKE, ws, NULL) ==
         MUSE_ERR_INVALID_ARG);   /* beyond the block table */
  EXPECT(reached_device(muse_attn_decode(&p, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, &g, FAKE, FAKE, ws, NULL)));
  /* the allocation-free entry point rejects calls beyond its scratch before any device work */
  muse_kv_cache huge = paged(1 << 20, 32, (int64_t)1 << 30);
  EXPECT(muse_attn_decode_noalloc(&p, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 25, &huge, FAKE, NULL) ==
         MUSE_ERR_WORKSPACE);
}

static void block_checks(void) {
  const muse_attn_params p = spark_global();
  muse_block_weights w;
  memset(&w, 0, sizeof w);
  w.hidden = 8192;
  w.in_norm = FAKE;
  w.w_qkvg = FAKE;
  w.w_o = FAKE;
  w.residual_gate = (const float*)FAKE;
  w.residual_gate_temperature = 0.3f;
  EXPECT(muse_attn_block_prefill_workspace_size(&p, &w, 1, 4096) > 0);
  EXPECT(muse_attn_block_prefill_workspace_size(&p, NULL, 1, 4096) == 0);
  muse_block_weights wb = w;
  wb.hidden = 100;   /* not a multiple of 8 */
  EXPECT(muse_attn_block_prefill_workspace_size(&p, &wb, 1, 4096) == 0);
  wb.hidden = -8;
  EXPECT(muse_attn_block_prefill_workspace_size(&p, &wb, 1, 4096) == 0);
  const size_t ws = muse_attn_block_prefill_workspace_size(&p, &w, 1, 4096);
  EXPECT(muse_attn_block_prefill(&p, &w, 1, 4096, NULL, FAKE, FAKE, ws, NULL) == MUSE_ERR_INVALID_ARG);
  EXPECT(muse_attn_block_prefill(&p, &w, 1, 4096, FAKE, FAKE, FAKE, ws - 1, NULL) == MUSE_ERR_WORKSPACE);
  EXPECT(reached_device(muse_attn_block_prefill(&p, &w, 1, 4096, FAKE, FAKE, FAKE, ws, NULL)));
}

int main(void) {
  workspace_sizes();
  prefill_checks();
  chunk_and_draft_checks();
  decode_checks();
  block_checks();
  for (int n = 1; n <= 96; ++n)
    for (int i = -1; i <= n; ++i) (void)muse_layer_is_global(i, n);
  EXPECT(muse_version() > 0);
  EXPECT(muse_profile_events(NULL, NULL) == MUSE_OK);
  if (fails) {
    printf("FAILED %d\n", fails);
    return 1;
  }
  printf("OK\n");
  return 0;
}
