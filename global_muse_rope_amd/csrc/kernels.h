// Kernel argument blocks, workspace layouts and host launchers.
#pragma once

#include "common.h"
#include "muse_attn.h"

namespace muse {

// Keys per LDS tile of the prefill kernel.
constexpr int kKeyTile = 64;

// ---------------------------------------------------------------------------
// Prefill workspace layouts (written by kv_prep_kernel, copied verbatim into
// LDS by the attention kernel, 16-byte chunks XOR-swizzled so that the MFMA
// operand reads of 32 consecutive rows spread over all LDS banks):
//   khat: fp16 [B * Hkv][n_tiles][64 keys][D], chunk c of key row r stored at
//         chunk k_chunk_swizzle(c, r);
//   vt:   bf16 [B * Hkv][n_tiles][D][64 keys], head-dim-major; inside each
//         16-key group keys are stored in the order 0-3, 8-11, 4-7, 12-15 so
//         that one 16-byte read gives the eight keys an MFMA lane consumes;
//         chunk c of dim row d stored at chunk v_chunk_swizzle(c, d).
// ---------------------------------------------------------------------------

// Rows of 128 bytes (8 chunks): XOR with ((d >> 1) & 7) ^ ((d & 1) << 2) gives
// distinct chunks to any 8 consecutive rows and, within the even and within
// the odd rows of any 16 consecutive rows, so 16-byte reads of 16 rows at one
// logical chunk hit distinct banks whether the LDS serves 8 or 16 lanes per
// cycle.
__host__ __device__ __forceinline__ int row128_swizzle(int d) { return ((d >> 1) & 7) ^ ((d & 1) << 2); }

template <int D>
__host__ __device__ __forceinline__ int k_chunk_swizzle(int c, int r) {
  return D == 128 ? (c ^ (r & 15)) : (c ^ row128_swizzle(r));
}

__host__ __device__ __forceinline__ int v_chunk_swizzle(int c, int d) { return c ^ row128_swizzle(d); }

struct RopeQkArgs {
  const uint16_t* x;
  int64_t stride_tok;
  int heads;
  int64_t n_rows;  // n_tokens * heads
  const int32_t* positions;
  float scale;
  float eps;
  double log2_theta;
  int use_rope;
  void* out;
};

// RoPE table: (cos, sin) of position * theta^(-2j/D) for j < D/2, float2
// [rows][D/2] with rows = T (positions 0..T-1) or B * T (explicit positions).
struct RopeTableArgs {
  const int32_t* positions;  // null: position = token index
  int T;
  int64_t n_rows;
  double log2_theta;
  float2* table;
};

struct KvPrepArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_sb, k_st, v_sb, v_st;
  const float2* rope;  // null on NoPE layers
  int rope_batched;    // table rows indexed by b * T + t (else t)
  int T, Hkv, n_tiles;
  float eps;
  half_t* khat;
  uint16_t* vt;
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* gate;
  uint16_t* out;
  const half_t* khat;
  const uint16_t* vt;
  int64_t q_sb, q_st, g_sb, g_st, o_sb, o_st;
  const float2* rope;  // null on NoPE layers
  int rope_batched;
  int T, Hkv, W, n_tiles, n_qblocks, n_qblocks_pad, batch_heads;
  float qscale;  // s * log2(e) / sqrt(D): logits come out in log2 units
  float qk_eps;
  int out_norm;
  float out_eps;
};

struct DecodeArgs {
  const uint16_t* q_new;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* gate;
  const int32_t* kv_len;
  uint16_t* out;
  // cache
  uint16_t* kc;
  uint16_t* vc;
  const int32_t* block_table;
  int kind, capacity, max_pages, page_tokens;
  int64_t num_pages;
  // shape
  int B, Hkv, W, max_kv_len;
  int chunk_tokens, max_chunks;
  float qscale, qk_eps, out_eps;
  double log2_theta;
  int use_rope, out_norm;
  // workspace
  float* qhat;    // [B, Hq, D] fp32, scaled into log2 units
  float* khat;    // [B, Hkv, D] fp32 new key
  float* part;    // [B * Hkv][max_chunks][G * (D + 2)] partial results
};

hipError_t launch_rope_qknorm(int d, int out_dtype, const RopeQkArgs& a, hipStream_t st);
hipError_t launch_rope_table(int d, const RopeTableArgs& a, hipStream_t st);
hipError_t launch_kv_prep(int d, int B, const KvPrepArgs& a, hipStream_t st);
hipError_t launch_prefill(int d, int g, const PrefillArgs& a, hipStream_t st);
int prefill_rows_per_block(int d, int g);
int prefill_qblock_group();
// ev0/ev1 (may be null): recorded around the split kernel.
hipError_t launch_decode(int d, int g, const DecodeArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace muse
