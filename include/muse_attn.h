/*
 * muse_attn.h - C ABI of the MI355X (gfx950) attention library for the
 * Muse Glimmer / Muse Spark Open attention layer.
 *
 * The layer (Muse Spark Open deep dive, gangliao.me, section 3 and its
 * subsections 3.1-3.4; the normalization-and-gates audit on flozi.net):
 *   - grouped-query attention, query head h reads KV head floor(h / G),
 *     G = num_q_heads / num_kv_heads (section 3.1);
 *   - weightless per-head RMS norm of q and k, x / sqrt(mean(x^2) + eps),
 *     then q multiplied by the fixed qk_scale_factor, logits keep the usual
 *     1/sqrt(D) (section 3.2, the five-step forward order);
 *   - RoPE only on local layers: dimension j paired with j + D/2, angle
 *     position * theta^(-2j/D); global layers are NoPE (section 3.4);
 *   - causal mask: key j visible to query i iff j <= i and, on a local layer
 *     with window W, j > i - W (section 3.4, mask note);
 *   - Spark only: weightless RMS norm of each head's D outputs, then for both
 *     models the elementwise gate y = o * sigmoid(g) (section 3.3).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP device memory) unless a
 *     parameter says "host".  Tensors are bf16 unless stated.  Within one
 *     head a vector of D elements is contiguous; heads of one token are
 *     contiguous (head stride D).  Pointers must be 16-byte aligned and
 *     token/batch strides multiples of 8 elements.
 *   - The caller owns and allocates every buffer, including the workspace;
 *     the library allocates and frees nothing and keeps no device state
 *     between calls.  `stream` is a hipStream_t (0 = the null stream).
 *   - Every argument check runs on the host before any launch; on failure
 *     nothing is enqueued and the call returns a status code, with a message
 *     available from muse_last_error() (thread-local).  Calls are
 *     asynchronous: success means the work was enqueued on `stream`.
 *   - Supported shapes: head_dim 64 or 128; num_q_heads a multiple of
 *     num_kv_heads with G = num_q_heads / num_kv_heads in {1, 2, 4, 8, 16};
 *     the device must be gfx950.
 */
#ifndef MUSE_ATTN_H
#define MUSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muse_status {
  MUSE_OK = 0,
  MUSE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, stride or alignment */
  MUSE_ERR_UNSUPPORTED = 2,   /* head_dim, group size or device arch not supported */
  MUSE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the size query */
  MUSE_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} muse_status;

enum { MUSE_DTYPE_BF16 = 0, MUSE_DTYPE_F16 = 1, MUSE_DTYPE_F32 = 2, MUSE_DTYPE_FP8_E4M3 = 3 };
enum { MUSE_KV_RING = 0, MUSE_KV_PAGED = 1 };

/* One attention layer's settings, named after the models' config keys
 * (deep dive, section 1.2 table): num_attention_heads, num_key_value_heads,
 * head_dim, sliding_window, layer_rope_theta, qk_scale_factor, rms_norm_eps. */
typedef struct muse_attn_params {
  int32_t num_q_heads;    /* Hq: 32 (Glimmer) or 128 (Spark) */
  int32_t num_kv_heads;   /* Hkv: 2 (Glimmer) or 16 (Spark) */
  int32_t head_dim;       /* D: 128 (Glimmer) or 64 (Spark) */
  int32_t sliding_window; /* W > 0: local layer; 0: global layer (full causal) */
  float rope_theta;       /* RoPE base; 0 = NoPE (no rotation), as layer_rope_theta */
  float qk_scale;         /* query multiplier s: 3.87 or 5.4730064863875 */
  float qk_norm_eps;      /* eps of the weightless QK-norm, 1e-5 */
  int32_t out_norm;       /* 1: per-head weightless output RMS norm (Spark); 0: none */
  float out_norm_eps;     /* eps of the output norm */
} muse_attn_params;

/* Caller-owned KV cache of one layer, holding keys AFTER norm and RoPE (the
 * cache is updated after those steps: deep dive, section 3.2 notes).
 *
 * MUSE_KV_RING (local layers): k is [B, Hkv, capacity, D]; v is stored
 *   transposed per head, [B, Hkv, D, capacity].  Position p lives in slot
 *   p mod capacity; capacity must equal the layer's window W, so once the
 *   new token is written the ring holds exactly the W visible entries.
 * MUSE_KV_PAGED (global layers): a pool of pages, each page holding
 *   page_tokens consecutive positions of every KV head.  k is
 *   [num_pages, Hkv, page_tokens, D]; v is [num_pages, Hkv, D, page_tokens].
 *   Position p of sequence b lives in page block_table[b * max_pages_per_seq
 *   + p / page_tokens], row p mod page_tokens.  With D = 64 and
 *   page_tokens = 32 each (page, head) slice of K (or V) is 4 KiB in bf16.
 * V is head-dim-major inside a page (and inside a ring head) so that both
 * contractions read contiguous runs along their reduction axis.
 *
 * Element type (dtype):
 *   MUSE_DTYPE_BF16: entries are bf16; k_scale and v_scale are ignored.
 *   MUSE_DTYPE_FP8_E4M3: entries are OCP E4M3 codes (one byte: sign, 4
 *     exponent bits with bias 7, 3 mantissa bits, subnormals, 0x7F/0xFF NaN,
 *     largest magnitude 448).  A stored value x is the code of x / scale,
 *     the division in fp32, rounded to nearest with ties to an even mantissa
 *     and saturated to +-448; it reads back as value(code) * scale.  The
 *     scales are fp32 device arrays the caller owns and sets: k_scale and
 *     v_scale are [num_pages, Hkv] for PAGED (one per page and KV head) and
 *     [B, Hkv] for RING (one per sequence and KV head).  The pages size an
 *     FP8 cache and leave scale factors out (deep dive, section 7.2); this
 *     convention is the library's own. */
typedef struct muse_kv_cache {
  int32_t kind;                /* MUSE_KV_RING or MUSE_KV_PAGED */
  int32_t capacity;            /* RING: entries per (sequence, head); must equal W */
  void* k;                     /* device, dtype */
  void* v;                     /* device, dtype */
  const int32_t* block_table;  /* PAGED: device int32 [B, max_pages_per_seq] */
  int32_t max_pages_per_seq;   /* PAGED: row length of block_table */
  int32_t page_tokens;         /* PAGED: positions per page, a multiple of 16 */
  int64_t num_pages;           /* PAGED: pages in the pool (block_table entries must be < this) */
  int32_t dtype;               /* MUSE_DTYPE_BF16 (0) or MUSE_DTYPE_FP8_E4M3 */
  const float* k_scale;        /* FP8 only: device fp32, see above */
  const float* v_scale;        /* FP8 only: device fp32, see above */
} muse_kv_cache;

/* muse_rope_qknorm: the layer's prologue on its own (deep dive, section 3.2
 * steps 2-4 and section 3.4).
 *   q_hat = s * q / sqrt(mean(q^2) + eps), k_hat = k / sqrt(mean(k^2) + eps),
 *   then, if rope_theta != 0, both rotated by their token's position.
 * q: [n_tokens, Hq, D] bf16 with token stride q_stride_tok (elements);
 * k: [n_tokens, Hkv, D] bf16 with token stride k_stride_tok;
 * positions: device int32 [n_tokens], or NULL for 0 .. n_tokens-1;
 * q_out: [n_tokens, Hq, D], k_out: [n_tokens, Hkv, D], contiguous, in
 *   out_dtype (MUSE_DTYPE_BF16, _F16 or _F32), rounded to nearest even.
 * Either q (with q_out) or k (with k_out) may be NULL to process only the
 * other.  n_tokens == 0 is a no-op. */
int32_t muse_rope_qknorm(const muse_attn_params* params, int32_t n_tokens,
                         const void* q, int64_t q_stride_tok,
                         const void* k, int64_t k_stride_tok,
                         const int32_t* positions,
                         void* q_out, void* k_out, int32_t out_dtype,
                         void* stream);

/* muse_attn_prefill: the whole layer over B causal sequences of T tokens
 * (section 3.2 forward order, the mask of section 3.4 and the gate and
 * output norm of section 3.3), after the q/k/v/gate projections and before
 * o_proj.
 * q, gate: [B, T, Hq, D]; k, v: [B, T, Hkv, D]; out: [B, T, Hq, D]; bf16.
 * strides: host int64[10] = {batch, token} strides in elements of q, k, v,
 *   gate, out in that order, or NULL for contiguous tensors.
 * positions: device int32 [B, T] RoPE positions, or NULL for 0 .. T-1.  The
 *   mask always uses the token index inside the sequence.
 * workspace: device scratch of at least muse_attn_prefill_workspace_size()
 *   bytes (16-byte aligned), clobbered by the call.
 * T == 0 or B == 0 is a no-op. */
int32_t muse_attn_prefill(const muse_attn_params* params, int32_t B, int32_t T,
                          const void* q, const void* k, const void* v, const void* gate,
                          const int64_t* strides, const int32_t* positions,
                          void* out, void* workspace, size_t ws_bytes, void* stream);

size_t muse_attn_prefill_workspace_size(const muse_attn_params* params, int32_t B, int32_t T);

/* muse_attn_prefill_chunk: chunked prefill.  Each of B sequences continues
 * with a chunk of T new tokens after start[b] positions already held in a
 * KV cache (the step beside decode that fills the caches decode reads:
 * deep dive, section 7.2 on chunked prefill with KV reuse, and section 3.4
 * for the window the ring keeps).
 * Chunk token t of sequence b sits at position P = start[b] + t (RoPE angle
 * and mask).  Its query sees the visible positions of section 3.4's mask:
 * cached ones below start[b], read as stored (bf16, or E4M3 code times its
 * scale), and the chunk's own keys from start[b] to P, normalized and
 * rotated in fp32 like a whole-sequence prefill.  After the attention the
 * call writes the chunk's keys (bf16, or the E4M3 code of key / scale) and
 * values into the cache in place: a PAGED cache gets every position (its
 * block table must map pages for positions up to start[b] + T - 1; entries
 * outside [0, num_pages) are skipped and read as zeros), a RING the last
 * min(T, W) positions at slot p mod W.
 * q, gate: [B, T, Hq, D]; k, v: [B, T, Hkv, D]; out: [B, T, Hq, D]; bf16.
 * strides: host int64[10] as for muse_attn_prefill, or NULL.
 * start: device int32 [B]; each start[b] must lie in [0, max_start]: a
 *   sequence outside that range gets zero output and no cache write.  On a
 *   local layer the cache must hold positions max(0, start[b] - W + 1) ..
 *   start[b] - 1, on a global layer 0 .. start[b] - 1.
 * max_start: host bound on start (sizes the workspace); for a PAGED cache
 *   max_start + T must not exceed max_pages_per_seq * page_tokens.
 * cache: as for muse_attn_decode (a RING needs capacity == W).
 * workspace: at least muse_attn_prefill_chunk_workspace_size() bytes; it
 *   holds a tile image of every sequence's visible history plus the chunk.
 * Cached keys are taken as stored and need not have unit RMS.  The softmax
 *   keeps no running maximum: its logits are bounded per query block by
 *   s * sqrt(D) * max(1, largest RMS of the block's cached key rows), and
 *   where that bound passes 96 (log2 units) every logit of the block is
 *   shifted down by the excess, so sums stay in fp32 range.  Outputs are
 *   exact (to rounding) for cached-key RMS up to about 2.5; beyond that a
 *   row whose every logit sits far below the bound can lose its weights to
 *   underflow.  Cached key elements must lie within fp16 range (|x| < 65504).
 * T == 0 or B == 0 is a no-op. */
int32_t muse_attn_prefill_chunk(const muse_attn_params* params, int32_t B, int32_t T,
                                const void* q, const void* k, const void* v, const void* gate,
                                const int64_t* strides, const int32_t* start, int32_t max_start,
                                const muse_kv_cache* cache, void* out,
                                void* workspace, size_t ws_bytes, void* stream);

size_t muse_attn_prefill_chunk_workspace_size(const muse_attn_params* params, int32_t B, int32_t T,
                                              int32_t max_start);

/* muse_attn_draft_block: the non-causal block attention of a
 * block-diffusion drafter (deep dive, section 8.2, the drafter's fourth
 * step).  Each of B sequences has start[b] context positions in the cache
 * and a block of T tokens at positions start[b] .. start[b] + T - 1.  The
 * block's queries attend to the cached context (as stored) followed by the
 * block's own keys and values, with no causal mask: key position j is
 * visible to query position P iff |P - j| < W on a layer with window W (both
 * directions), and on a window-0 layer always, keys existing up to the
 * block's last position.  The block is not written into the cache (a
 * drafter drops it before the next block).
 * Arguments as for muse_attn_prefill_chunk, except that the cache only
 * needs positions below start[b] (a PAGED cache: max_start <=
 * max_pages_per_seq * page_tokens) and is left unchanged; a start outside
 * [0, max_start] gives zero output.
 * Blocks of at most 64 tokens whose T * (Hq / Hkv) query columns number at
 * most 128 per KV head run as a few-token decode: the cache is read as
 * stored through LDS once per 64 columns, the softmax keeps a running
 * maximum (cached keys of any RMS give exact results; key elements need
 * only be finite), and the block's own keys are normalized and rotated in
 * fp32.  Wider blocks go through the prefill kernel as a chunk does,
 * including its bound on logits over cached keys.
 * workspace: at least muse_attn_draft_block_workspace_size() bytes (few-token
 * blocks: fp32 partial sums per context chunk; wider ones: the chunk's tile
 * images). */
int32_t muse_attn_draft_block(const muse_attn_params* params, int32_t B, int32_t T,
                              const void* q, const void* k, const void* v, const void* gate,
                              const int64_t* strides, const int32_t* start, int32_t max_start,
                              const muse_kv_cache* cache, void* out,
                              void* workspace, size_t ws_bytes, void* stream);

size_t muse_attn_draft_block_workspace_size(const muse_attn_params* params, int32_t B, int32_t T,
                                            int32_t max_start);

/* muse_attn_decode: one new token per sequence against a KV cache.
 * q_new, gate, out: [B, Hq, D]; k_new, v_new: [B, Hkv, D]; contiguous bf16.
 * kv_len: device int32 [B], the sequence length INCLUDING the new token;
 *   the new token's position is kv_len[b] - 1.  Every kv_len[b] must lie in
 *   [1, max_kv_len]; a sequence outside that range gets zero output and no
 *   cache write.
 * max_kv_len: host upper bound on kv_len (sizes the launch); for a PAGED
 *   cache it must not exceed max_pages_per_seq * page_tokens.
 * The call writes the new token's normalized (and, on local layers, rotated)
 * key and its value into the cache in place, then attends the query to the
 * visible cached entries plus the new token (global: positions 0 .. p;
 * local: p - W < j <= p).  The new token's own key and value enter the
 * softmax at full fp32 precision; cached entries as stored (bf16).
 * workspace: at least muse_attn_decode_workspace_size() bytes. */
int32_t muse_attn_decode(const muse_attn_params* params, int32_t B,
                         const void* q_new, const void* k_new, const void* v_new,
                         const void* gate, const int32_t* kv_len, int32_t max_kv_len,
                         const muse_kv_cache* cache, void* out,
                         void* workspace, size_t ws_bytes, void* stream);

size_t muse_attn_decode_workspace_size(const muse_attn_params* params, int32_t B,
                                       int32_t max_kv_len, const muse_kv_cache* cache);

/* muse_attn_decode_noalloc: muse_attn_decode without a workspace argument,
 * for callers that cannot allocate device memory around the call (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, layouts, results and cache update as
 * muse_attn_decode; the call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine).
 * Its scratch is a fixed device array inside the library of
 * MUSE_DECODE_NOALLOC_SCRATCH_BYTES (80 MiB) per device, held from the
 * library's first use on a device until the process ends.  A call whose
 * muse_attn_decode_workspace_size() exceeds that returns
 * MUSE_ERR_WORKSPACE before any launch.  (80 MiB holds the decode of 16
 * sequences x 16 KV heads of width 64 at lengths up to 2^20, 67 MiB.)
 * Every call on one device shares that device's array: calls that overlap
 * on one device (different streams, host threads) race and must be
 * serialized by the caller. */
#define MUSE_DECODE_NOALLOC_SCRATCH_BYTES (80u << 20)

int32_t muse_attn_decode_noalloc(const muse_attn_params* params, int32_t B,
                                 const void* q_new, const void* k_new, const void* v_new,
                                 const void* gate, const int32_t* kv_len, int32_t max_kv_len,
                                 const muse_kv_cache* cache, void* out, void* stream);

/* The attention half of one decoder block around the layer (deep dive,
 * section 2.1 forward walk; section 5.1 for Glimmer's sandwich norms, 5.2 for
 * Spark's norm-preserving residual gate, 5.3 for the RMSNorm variants):
 *   h   = x / sqrt(mean(x^2) + 1e-5) * (1 + in_norm)      input_layernorm
 *   q, k, v, gate = h W_q^T, h W_k^T, h W_v^T, h W_g^T     (no biases)
 *   o   = the layer (as muse_attn_prefill, positions 0 .. T-1)
 *   a   = o W_o^T                                         o_proj
 *   f   = a / sqrt(mean(a^2) + 1e-8), times (1 + post_norm) with a plain add
 *   out = x + f (residual_gate NULL), or alpha * x + beta * f with
 *         beta = sigmoid(g / T), alpha = sqrt(max(sigmoid(-g / T) (1 + beta), 1e-3))
 * Norm gains are formed and applied in fp32.  h enters the projection GEMM
 * as a pair of bf16 rows (h_hi = bf16(h), h_lo = bf16(h - h_hi): about 16
 * bits); the GEMMs take bf16 operands and accumulate and write fp32; the
 * layer receives q, k and the gate in fp16 and v in bf16 (the type of its
 * value product), and returns o in bf16; o_proj's output stays fp32 into the
 * post-norm and residual; the result is rounded once to bf16. */
typedef struct muse_block_weights {
  int32_t hidden;                  /* model width: 8192 (Spark) or 6656 (Glimmer); a multiple of 8, <= 8192 */
  const void* in_norm;             /* [hidden] bf16: input_layernorm weight w (gain 1 + w) */
  const void* w_qkvg;              /* [(2 Hq + 2 Hkv) D, hidden] bf16: rows of W_q, W_k, W_v, W_g stacked */
  const void* w_o;                 /* [hidden, Hq D] bf16 */
  const void* post_norm;           /* plain add: [hidden] bf16 post_attention_layernorm weight (gain 1 + w) */
  const float* residual_gate;      /* [hidden] fp32 residual-gate parameter g, or NULL for a plain add */
  float residual_gate_temperature; /* T, 0.3 */
} muse_block_weights;

/* muse_attn_block_prefill: the block's attention half over B sequences of T
 * tokens.  x, out: [B, T, hidden] bf16, contiguous.  The projections run as
 * hipBLASLt GEMMs on `stream` with the caller's workspace as their scratch.
 * Host state: the library keeps one hipBLASLt handle per device (created on
 * its first block call on that device) and, per device and GEMM shape, the
 * algorithm it runs: the one muse_attn_block_tune recorded, else hipBLASLt's
 * first heuristic choice (recorded at the first call of the shape).  Like
 * every other entry point except muse_attn_block_tune, the call never waits
 * for the device.
 * workspace: at least muse_attn_block_prefill_workspace_size() bytes.
 * T == 0 or B == 0 is a no-op. */
int32_t muse_attn_block_prefill(const muse_attn_params* params, const muse_block_weights* weights,
                                int32_t B, int32_t T, const void* x, void* out,
                                void* workspace, size_t ws_bytes, void* stream);

size_t muse_attn_block_prefill_workspace_size(const muse_attn_params* params,
                                              const muse_block_weights* weights, int32_t B, int32_t T);

/* muse_attn_block_decode: one new token per sequence through the block's
 * attention half (the same steps as muse_attn_block_prefill, deep dive
 * section 2.1 forward walk), with the layer as one decode step
 * (muse_attn_decode: the new token at position kv_len[b] - 1, its key and
 * value appended to `cache` in place, attention over the visible cached
 * entries plus itself).  x, out: [B, hidden] bf16, contiguous.  kv_len,
 * max_kv_len and cache as for muse_attn_decode; weights as for
 * muse_attn_block_prefill.  A sequence whose kv_len is out of range gets
 * only its residual term (its layer output is zero) and no cache write.
 * workspace: at least muse_attn_block_decode_workspace_size() bytes.
 * B == 0 is a no-op. */
int32_t muse_attn_block_decode(const muse_attn_params* params, const muse_block_weights* weights, int32_t B,
                               const void* x, const int32_t* kv_len, int32_t max_kv_len,
                               const muse_kv_cache* cache, void* out, void* workspace, size_t ws_bytes,
                               void* stream);

size_t muse_attn_block_decode_workspace_size(const muse_attn_params* params,
                                             const muse_block_weights* weights, int32_t B, int32_t max_kv_len,
                                             const muse_kv_cache* cache);

/* muse_attn_block_tune: optional, explicit tuning of the block's two
 * projection GEMMs for `rows` token rows (B * T for muse_attn_block_prefill,
 * B for muse_attn_block_decode) on the current device: times hipBLASLt's top
 * candidate algorithms on zeroed activations in the workspace and the given
 * weights, and records the fastest for the block calls that follow.  This
 * call WAITS for `stream` (it reads the timings back), so it belongs outside
 * timed or captured regions; the other entry points never wait.  Only
 * weights->hidden, w_qkvg and w_o are read.
 * workspace: at least muse_attn_block_prefill_workspace_size(params, weights,
 * 1, rows) bytes; its contents are clobbered. */
int32_t muse_attn_block_tune(const muse_attn_params* params, const muse_block_weights* weights, int32_t rows,
                             void* workspace, size_t ws_bytes, void* stream);

/* Layer schedule: layer i of n_layers is global (full attention, NoPE) iff
 * (n_layers - 1 - i) mod 4 == 0 (deep dive, section 2.2 equation).
 * Returns 1 (global), 0 (local) or -1 for i outside [0, n_layers). */
int32_t muse_layer_is_global(int32_t layer_index, int32_t n_layers);

/* Message of the last failed call on this thread ("" if none). */
const char* muse_last_error(void);

/* Profiling aid: on the calling thread, make the next muse_attn_prefill,
 * muse_attn_prefill_chunk, muse_attn_draft_block and muse_attn_decode calls
 * record `start` (a hipEvent_t) on their stream just before their main
 * attention kernel (the prefill attention kernel; the decode split kernel)
 * and `stop` just after it, so a caller can time that kernel with
 * hipEventElapsedTime.  A chunk or drafter call whose few query blocks are
 * split over key pieces records `stop` after the kernel that combines the
 * pieces.  Pass NULL, NULL to turn it off.  Nothing is recorded by
 * muse_rope_qknorm.  Returns MUSE_OK, or MUSE_ERR_INVALID_ARG if exactly one
 * of the two is NULL. */
int32_t muse_profile_events(void* start, void* stop);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t muse_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUSE_ATTN_H */
