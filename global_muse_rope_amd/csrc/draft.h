// The drafter's block attention over a cached context as a few-token decode:
// argument block, work split and launcher of the kernels in draft.hip.
#pragma once

#include <algorithm>

#include "kernels.h"

namespace muse {

// Blocks of at most kDraftMaxT tokens whose T * G query columns fit
// kDraftMaxCols per KV head take this path.  Each split workgroup covers
// kDraftGroupCols columns and reads its chunk of the cache once for them.
constexpr int kDraftMaxT = 64;
constexpr int kDraftMaxCols = 128;
constexpr int kDraftGroupCols = 64;
// Context chunk of one split workgroup: a multiple of 64 positions (its
// sub-chunks), at most kDraftChunkMax (its block table lives in LDS).
constexpr int kDraftChunkMax = 2048;
// Split workgroups aimed for: two per CU (each holds two 32 KB images of
// LDS and four waves).
constexpr int64_t kDraftWorkgroups = 512;

// A block of T tokens per sequence at positions start[b] .. start[b] + T - 1
// attends, with no causal mask, to the cached context below start[b] and to
// its own keys; key position j is visible to query position P iff
// |P - j| < W (every key when W = 0).  Query columns are (token, head) pairs
// of one KV head, column c = t * G + g for query head hk * G + g.
struct DraftArgs {
  // the block's q, k, v, gate [B, T, H, D] (bf16), {batch, token} strides in elements
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;
  int64_t q_sb, q_st, k_sb, k_st, v_sb, v_st, g_sb, g_st, o_sb, o_st;
  uint16_t* out;
  const int32_t* start;  // [B]; outside [0, max_start]: zero output
  int max_start;
  int B, T, Hkv, G, W;
  float qscale;  // s * log2(e) / sqrt(D): logits come out in log2 units
  float qk_eps, out_eps;
  int out_norm;
  double log2_theta;
  int use_rope;
  CacheView cache;
  // split over the context: chunks of chunk_tokens positions from
  // draft_ctx_base(start, W), one per workgroup, n_wg >= 1 workgroups per
  // (sequence, KV head, group of 64 columns)
  int chunk_tokens, n_cgroups, n_wg;
  // [B * Hkv][n_cgroups][n_wg][64][D + 4] floats: O, running max, sum (rows
  // 16-byte aligned); the last workgroup of a sequence adds the block's own
  // keys to its partial
  float* part;
};

// First position of a sequence's first context chunk: its first visible
// cached position rounded down to a multiple of 32.
__host__ __device__ inline int draft_ctx_base(int start, int W) {
  const int lo = W > 0 && start - W + 1 > 0 ? start - W + 1 : 0;
  return (lo / 32) * 32;
}

struct DraftPlan {
  int chunk_tokens, n_cgroups, n_wg;
};

// Whether a layer and block size take the split path.
inline bool draft_split_fits(int T, int G) { return T <= kDraftMaxT && static_cast<int64_t>(T) * G <= kDraftMaxCols; }

// Chunking for B sequences with starts up to max_start: start - base is at
// most W + 30 on a local layer (the base is rounded down to 32) and at most
// max_start.  At least one workgroup per (sequence, KV head, column group):
// the last one with context, or workgroup 0, also takes the block's own keys.
inline DraftPlan draft_plan(int B, int Hkv, int G, int T, int W, int max_start) {
  DraftPlan p;
  p.n_cgroups = (T * G + kDraftGroupCols - 1) / kDraftGroupCols;
  const int64_t ctx = W > 0 ? std::min<int64_t>(max_start, W + 30) : max_start;
  // chunks sized on the usual context (W on a local layer) plus the block's
  // own keys (about two sub-chunks of work, taken by the last workgroup with
  // context), so that the work splits evenly over about kDraftWorkgroups
  // workgroups; a longer context gets a short extra chunk, dispatched last
  const int64_t nominal = (W > 0 ? std::min<int64_t>(max_start, W) : max_start) + 128;
  const int64_t pairs = std::max<int64_t>(1, static_cast<int64_t>(B) * Hkv * p.n_cgroups);
  const int64_t want = std::max<int64_t>(1, kDraftWorkgroups / pairs);
  int64_t ct = (nominal + want - 1) / want;
  ct = std::min<int64_t>(kDraftChunkMax, std::max<int64_t>(64, (ct + 63) / 64 * 64));
  p.chunk_tokens = static_cast<int>(ct);
  p.n_wg = static_cast<int>(std::max<int64_t>(1, (ctx + ct - 1) / ct));
  return p;
}

hipError_t launch_draft(int d, const DraftArgs& a, hipStream_t st);

}  // namespace muse
