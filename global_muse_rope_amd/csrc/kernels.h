// Kernel argument blocks, workspace layouts and host launchers.
#pragma once

#include "common.h"
#include "muse_attn.h"

namespace muse {

// Keys per LDS tile of the prefill kernel.
constexpr int kKeyTile = 64;
// Cached positions per split workgroup of a paged decode cache: the largest
// of kPagedChunkMax, its half and its quarter for which a launch still has
// kPagedChunkTarget workgroups or more (the smallest otherwise).
constexpr int kPagedChunkMax = 8192;
constexpr int kPagedChunkMin = 2048;
constexpr int64_t kPagedChunkTarget = 2048;

// ---------------------------------------------------------------------------
// Prefill tile image: one 64-key tile of one (sequence, KV head), written by
// kv_prep_kernel and copied verbatim into LDS by the attention kernel, in
// 16-byte chunks:
//   K part: 64 key rows of k_hat (fp16), D/8 chunks each;
//   V part: D head-dim rows of V (bf16) over the 64 keys, 8 chunks each;
//           inside each 16-key group the keys are stored in the order 0-3,
//           8-11, 4-7, 12-15 so that one 16-byte read gives the eight keys an
//           MFMA lane consumes.
// Both parts are chunk-major: chunk c of every row, then chunk c + 1.  Lanes
// that read one chunk of consecutive rows then touch consecutive 16-byte
// chunks (16 distinct bank groups per 16 lanes, with no pad chunks), and
// every MFMA fragment address is an immediate offset from one per-lane base.
// ---------------------------------------------------------------------------
template <int D>
struct TileLayout {
  static constexpr int KCHUNKS = kKeyTile * (D / 8);
  static constexpr int VCHUNKS = D * (kKeyTile / 8);
  static constexpr int CHUNKS = KCHUNKS + VCHUNKS;
  static_assert(CHUNKS % 64 == 0, "a tile is copied in whole 64-lane wave instructions");
  // chunk index of chunk c (head dims 8c .. 8c + 7) of key row r
  __host__ __device__ static constexpr int k(int r, int c) { return c * kKeyTile + r; }
  // chunk index of chunk c (eight keys, in the order above) of head-dim row d
  __host__ __device__ static constexpr int v(int d, int c) { return KCHUNKS + c * D + d; }
};

inline int tile_chunks(int d) { return d == 128 ? TileLayout<128>::CHUNKS : TileLayout<64>::CHUNKS; }

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
  const int32_t* start;      // chunked prefill: position of row b * T + t is start[b] + t
  int max_start;             // start values outside [0, max_start] count as 0
  int T;
  int64_t n_rows;
  double log2_theta;
  float2* table;
};

// ---------------------------------------------------------------------------
// Chunked prefill: a chunk of T tokens at positions start .. start + T - 1
// continues a sequence whose first `start` positions are cached.  The tile
// image of sequence b covers key slots s = position - kbase(start, W): local
// layers start at the window's first position rounded down to a tile, global
// layers at position 0.  Tiles stay aligned to positions, and query row t of
// the chunk is key slot t + start - kbase.
// ---------------------------------------------------------------------------
__host__ __device__ inline int chunk_kbase(int start, int W) {
  const int lo = start - W + 1;
  return W > 0 && lo > 0 ? (lo / kKeyTile) * kKeyTile : 0;
}
__host__ __device__ inline bool chunk_start_ok(int start, int max_start) {
  return start >= 0 && start <= max_start;
}

// A layer's KV cache as the kernels see it (element offsets are the same for
// bf16 entries and E4M3 codes; the byte size differs).
struct CacheView {
  int kind, capacity, max_pages, page_tokens;
  int64_t num_pages;
  const int32_t* block_table;
  void* k;
  void* v;
  int fp8;
  const float* k_scale;  // fp8: [num_pages, Hkv] (paged) or [B, Hkv] (ring)
  const float* v_scale;
};

struct KvPrepArgs {
  const uint16_t* k;  // bf16, or fp16 when k_f16 (v is always bf16)
  const uint16_t* v;
  int k_f16;
  int64_t k_sb, k_st, v_sb, v_st;
  const float2* rope;  // null on NoPE layers
  int rope_batched;    // table rows indexed by b * T + t (else t)
  int T, Hkv, n_tiles;
  float eps;
  u32x4* tiles;        // [B * Hkv][n_tiles][TileLayout<D>::CHUNKS]
  // chunked prefill (start != null): slot s of sequence b is position
  // chunk_kbase(start[b], W) + s; cached positions come from `cache`
  const int32_t* start;
  int max_start, W;
  CacheView cache;
  // chunked prefill: per tile, the largest mean square of its cached key
  // rows as the attention will read them (0 for a tile without any),
  // [B * Hkv][n_tiles]; every tile's entry is written
  float* tile_ms;
};

// Writes a chunk's normalized (and rotated) keys and its values into the
// cache: every position of a paged cache, the last min(T, W) of a ring.
struct ChunkAppendArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_sb, k_st, v_sb, v_st;
  const float2* rope;  // rows b * T + t, null on NoPE layers
  const int32_t* start;
  int max_start, T, Hkv, W;
  float eps;
  CacheView cache;
};

struct PrefillArgs {
  const uint16_t* q;     // q and gate: bf16, or fp16 when in_f16
  const uint16_t* gate;
  int in_f16;
  uint16_t* out;
  const u32x4* tiles;  // [B * Hkv][n_tiles][TileLayout<D>::CHUNKS]
  int64_t q_sb, q_st, g_sb, g_st, o_sb, o_st;
  const float2* rope;  // null on NoPE layers
  int rope_batched;
  int T, Hkv, W, n_tiles, n_qblocks, n_qblocks_pad, batch_heads;
  float qscale;  // s * log2(e) / sqrt(D): logits come out in log2 units
  float qk_eps;
  int out_norm;
  float out_eps;
  // chunked prefill (null otherwise): query row t of sequence b is key slot
  // t + start[b] - chunk_kbase(start[b], W); a start outside [0, max_start]
  // gives zero output rows
  const int32_t* start;
  int max_start;
  // 1: no causal mask; key slot j is visible to query slot i iff |i - j| < W
  // (every key on a window-0 layer), up to the last key slot
  int noncausal;
  // key split (nsplit > 1): workgroup x takes query block x / nsplit and the
  // (x mod nsplit)-th of nsplit contiguous pieces of that block's tile range,
  // and writes unnormalized partial sums for the combine kernel instead of
  // outputs: part_o [nsplit][B][T][Hq][D] (sum of p v) and part_l
  // [nsplit][B][T][Hq] (sum of p); an empty piece writes zeros
  int nsplit;
  float* part_o;
  float* part_l;
  // chunked prefill and drafter blocks (null otherwise): per-tile largest
  // mean square of the cached key rows ([B * Hkv][n_tiles], kv_prep).  A
  // block's logits are then bounded by qbound * sqrt(max(1, that maximum))
  // in log2 units (qbound = qscale * D); where that bound exceeds
  // kLogitCap, every logit of the block is shifted down by the excess, so
  // no exponential or sum leaves fp32 range.
  const float* tile_ms;
  float qbound;
};

// Largest exponent (log2 units) the max-free softmax lets a logit reach
// before a block-wide shift applies: 2^96 times 2^20 keys stays below
// fp32's range with room for |v| up to 2^11.
constexpr float kLogitCap = 96.0f;

// Finishes a key-split prefill: sums the partials of each output row, then
// 1/sum, the per-head output norm, the sigmoid gate and the bf16 store.
struct PrefillCombineArgs {
  const float* part_o;
  const float* part_l;
  int nsplit;
  const uint16_t* gate;
  uint16_t* out;
  int64_t g_sb, g_st, o_sb, o_st;
  int B, T, Hq;
  int out_norm;
  float out_eps;
  const int32_t* start;  // rows of a sequence whose start is out of range are zero
  int max_start;
};

struct DecodeArgs {
  int in_f16;             // q_new, k_new and gate in fp16 instead of bf16 (v_new is always bf16)
  const uint16_t* q_new;  // [B, Hq, D] with batch stride q_sb (elements)
  const uint16_t* k_new;  // [B, Hkv, D] with batch stride kv_sb
  const uint16_t* v_new;  // [B, Hkv, D] with batch stride kv_sb
  const uint16_t* gate;   // [B, Hq, D] with batch stride g_sb
  int64_t q_sb, kv_sb, g_sb;
  const int32_t* kv_len;
  uint16_t* out;
  // cache (bf16 entries, or E4M3 codes when fp8 is set; element offsets
  // are the same, the byte size differs)
  uint16_t* kc;
  uint16_t* vc;
  int fp8;
  const float* k_scale;  // fp8: [num_pages, Hkv] (paged) or [B, Hkv] (ring)
  const float* v_scale;
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

// ---------------------------------------------------------------------------
// The attention half of a decoder block: row kernels around two GEMMs.
// ---------------------------------------------------------------------------
constexpr int kBlockMaxHidden = 8192;

struct BlockNormArgs {
  const uint16_t* x;  // [rows, hidden] bf16
  const uint16_t* w;  // [hidden] bf16 weight (gain 1 + w)
  uint16_t* out;      // [rows, hidden] bf16: h rounded to bf16 (h_hi)
  uint16_t* out_lo;   // [rows, hidden] bf16: h - h_hi rounded to bf16
  int64_t rows;
  int hidden;
  float eps;
};

// The projections' sum over the hi and lo halves of h, handed to the layer:
// proj [2 rows, n] fp32 (rows of h_hi W^T, then rows of h_lo W^T) -> out
// [rows, n] 16-bit: q, k and gate columns in fp16, v columns in bf16.
struct BlockProjPrepArgs {
  const float* proj;
  uint16_t* out;
  int64_t rows;
  int n, q_end, k_end, v_end;  // column ranges [0, q_end) q, [q_end, k_end) k, [k_end, v_end) v, then gate
};

struct BlockResidualArgs {
  const uint16_t* x;          // residual stream [rows, hidden] bf16
  const float* branch;        // o_proj output [rows, hidden] fp32
  const uint16_t* post_norm;  // plain add: [hidden] bf16 weight (gain 1 + w)
  const float* coef;          // residual gate: [hidden] (alpha, beta) fp32 pairs (null: plain add)
  uint16_t* out;
  int64_t rows;
  int hidden;
  float eps;
};

hipError_t launch_block_input_norm(const BlockNormArgs& a, hipStream_t st);
hipError_t launch_block_proj_prep(const BlockProjPrepArgs& a, hipStream_t st);
hipError_t launch_block_residual(const BlockResidualArgs& a, hipStream_t st);
// (alpha, beta) of the residual gate for every channel of g
hipError_t launch_block_gate_coef(const float* gate, float2* coef, int hidden, float temperature,
                                  float alpha_sq_floor, hipStream_t st);
// out[rows, n] = act[rows, k] * w[n, k]^T (bf16 operands, fp32 accumulation,
// fp32 out); returns 0, or non-zero with a message in err.  tune: time the top
// candidate algorithms (waits for the stream) and record the fastest for this
// shape.
int block_gemm(int64_t rows, int64_t n, int64_t k, const void* act, const void* w, float* out, void* ws,
               size_t ws_bytes, hipStream_t st, char* err, size_t errlen, bool tune = false);

hipError_t launch_rope_qknorm(int d, int out_dtype, const RopeQkArgs& a, hipStream_t st);
hipError_t launch_rope_table(int d, const RopeTableArgs& a, hipStream_t st);
hipError_t launch_kv_prep(int d, int B, const KvPrepArgs& a, hipStream_t st);
hipError_t launch_chunk_append(int d, int B, const ChunkAppendArgs& a, hipStream_t st);
hipError_t launch_prefill(int d, int g, const PrefillArgs& a, hipStream_t st);
int prefill_rows_per_block(int d, int g);
// Key pieces per query block for a launch of n_blocks query blocks whose
// blocks span at most max_tiles key tiles on a device of `cus` compute units:
// 1 when the blocks alone fill the chip, else enough pieces for about one
// workgroup per CU, each of at least two tiles (at most 16 pieces).
int prefill_key_split(int64_t n_blocks, int64_t max_tiles, int cus);
hipError_t launch_prefill_combine(int d, const PrefillCombineArgs& a, hipStream_t st);
int prefill_qblock_group();
// ev0/ev1 (may be null): recorded around the split kernel.
hipError_t launch_decode(int d, int g, const DecodeArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace muse
