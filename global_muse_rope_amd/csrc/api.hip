// C ABI: host-side argument checks, workspace sizing and kernel dispatch.
// Every check runs before any launch; the library keeps no device state.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "draft.h"
#include "kernels.h"

using namespace muse;

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode entry point (muse_attn_decode_noalloc):
// one array per device, held from the library's first use on that device
// until the process ends.  On the host the name is a stand-in, not device
// memory: host code passes only the device address hipGetSymbolAddress
// returns for it.  Every value a call reads from it is written earlier in
// the same call, so nothing is cleared between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MUSE_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return MUSE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_arch_mu;
int g_arch_state[kMaxDevices] = {0};  // 0 unknown, 1 gfx950, 2 other

int32_t check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MUSE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_arch_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  if (g_arch_state[dev] != 1) return fail(MUSE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return MUSE_OK;
}

bool pow2_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

int32_t check_params(const muse_attn_params* p) {
  if (!p) return fail(MUSE_ERR_INVALID_ARG, "params is NULL");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(MUSE_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(MUSE_ERR_INVALID_ARG, "head counts must be positive");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(MUSE_ERR_UNSUPPORTED, "num_q_heads %d not a multiple of num_kv_heads %d", p->num_q_heads,
                p->num_kv_heads);
  if (!pow2_group(p->num_q_heads / p->num_kv_heads))
    return fail(MUSE_ERR_UNSUPPORTED, "group size %d not in {1,2,4,8,16}", p->num_q_heads / p->num_kv_heads);
  if (p->sliding_window < 0) return fail(MUSE_ERR_INVALID_ARG, "sliding_window must be >= 0");
  if (!(p->rope_theta >= 0.f) || !std::isfinite(p->rope_theta) || (p->rope_theta > 0.f && p->rope_theta <= 1.f))
    return fail(MUSE_ERR_INVALID_ARG, "rope_theta must be 0 (NoPE) or > 1");
  if (!std::isfinite(p->qk_scale) || p->qk_scale <= 0.f) return fail(MUSE_ERR_INVALID_ARG, "qk_scale must be > 0");
  if (!(p->qk_norm_eps > 0.f) || !std::isfinite(p->qk_norm_eps))
    return fail(MUSE_ERR_INVALID_ARG, "qk_norm_eps must be > 0");
  if (p->out_norm != 0 && p->out_norm != 1) return fail(MUSE_ERR_INVALID_ARG, "out_norm must be 0 or 1");
  if (p->out_norm && (!(p->out_norm_eps > 0.f) || !std::isfinite(p->out_norm_eps)))
    return fail(MUSE_ERR_INVALID_ARG, "out_norm_eps must be > 0");
  return MUSE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

double log2_theta(const muse_attn_params* p) {
  return p->rope_theta > 0.f ? std::log2(static_cast<double>(p->rope_theta)) : 0.0;
}

// s * log2(e) / sqrt(D): q_hat pre-multiplied so logits come out in log2 units.
float q_logit_scale(const muse_attn_params* p) {
  return static_cast<float>(static_cast<double>(p->qk_scale) * 1.4426950408889634 /
                            std::sqrt(static_cast<double>(p->head_dim)));
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Compute units of the current device (cached per device), or the MI355X's
// 256 where no device is visible (a workspace-size query on a host without a
// GPU); the key split of a chunk launch aims at one workgroup per CU.
int device_cus() {
  static int cached[kMaxDevices] = {};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  cached[dev] = n;
  return n;
}

int64_t prefill_tiles(int32_t T) { return (static_cast<int64_t>(T) + kKeyTile - 1) / kKeyTile; }

// Prefill workspace: the K/V tile images (k_hat fp16 + V^T bf16, padded rows)
// and, on RoPE layers, the (cos, sin) table for B * T positions.
struct PrefillWs {
  size_t tile_bytes, rope_bytes, part_o_bytes, part_l_bytes, tile_ms_bytes, total;
  int nsplit;
};

PrefillWs prefill_ws_layout(const muse_attn_params* p, int32_t B, int32_t T) {
  PrefillWs w;
  w.tile_bytes = align256(static_cast<size_t>(B) * p->num_kv_heads * prefill_tiles(T) * tile_chunks(p->head_dim) * 16);
  w.rope_bytes = p->rope_theta > 0.f ? align256(static_cast<size_t>(B) * T * (p->head_dim / 2) * 8) : 0;
  w.part_o_bytes = w.part_l_bytes = w.tile_ms_bytes = 0;
  w.nsplit = 1;
  w.total = w.tile_bytes + w.rope_bytes;
  return w;
}

size_t prefill_ws(const muse_attn_params* p, int32_t B, int32_t T) { return prefill_ws_layout(p, B, T).total; }

// Chunked prefill: tiles per sequence cover slots 0 .. start - kbase + T - 1,
// at most W - 1 + 63 slots of history on a local layer (the window's first
// position rounded down to a tile) and max_start on a global one.
int64_t chunk_tiles(const muse_attn_params* p, int32_t T, int32_t max_start) {
  const int64_t W = p->sliding_window;
  const int64_t hist = W > 0 ? std::min<int64_t>(max_start, W - 1 + kKeyTile - 1) : max_start;
  return (hist + T + kKeyTile - 1) / kKeyTile;
}

// Query blocks of a chunk launch (every sequence and KV head).
int64_t chunk_qblocks(const muse_attn_params* p, int32_t B, int32_t T) {
  const int G = p->num_q_heads / p->num_kv_heads;
  const int bq = prefill_rows_per_block(p->head_dim, G) / G;
  return (static_cast<int64_t>(T) + bq - 1) / bq * B * p->num_kv_heads;
}

// Tile images and the RoPE table, then, when the launch has too few query
// blocks to fill the chip (a short chunk or a drafter's block), the key
// pieces' partial sums: O fp32 [nsplit][B][T][Hq][D] and sums [..][Hq];
// last the per-tile largest cached-key mean square, fp32 [B][Hkv][n_tiles].
PrefillWs chunk_ws_layout(const muse_attn_params* p, int32_t B, int32_t T, int32_t max_start) {
  PrefillWs w;
  const int64_t n_tiles = chunk_tiles(p, T, max_start);
  w.tile_bytes = align256(static_cast<size_t>(B) * p->num_kv_heads * n_tiles * tile_chunks(p->head_dim) * 16);
  w.rope_bytes = p->rope_theta > 0.f ? align256(static_cast<size_t>(B) * T * (p->head_dim / 2) * 8) : 0;
  w.nsplit = prefill_key_split(chunk_qblocks(p, B, T), n_tiles, device_cus());
  const size_t rows = static_cast<size_t>(B) * T * p->num_q_heads;
  w.part_o_bytes = w.nsplit > 1 ? align256(w.nsplit * rows * p->head_dim * 4) : 0;
  w.part_l_bytes = w.nsplit > 1 ? align256(w.nsplit * rows * 4) : 0;
  w.tile_ms_bytes = align256(static_cast<size_t>(B) * p->num_kv_heads * n_tiles * 4);
  w.total = w.tile_bytes + w.rope_bytes + w.part_o_bytes + w.part_l_bytes + w.tile_ms_bytes;
  return w;
}

struct DecodePlan {
  int chunk_tokens;
  int max_chunks;
};

// Ring entries per split workgroup: a 2048-entry ring splits in two, which
// measured fastest on a cold cache (256: 11 %, 512: 8 %, 2048: 9 % slower).
constexpr int kRingChunk = 1024;
// Paged chunks: 8192 entries (512 KB of a bf16 cache at head width 64) per
// workgroup measured 3 % faster than 2048 on 16 sequences of up to 2^20
// positions, and 8 % faster on an E4M3 cache, mostly from fewer partials and
// fewer workgroup starts; 16384 was slower.  Small batches of short sequences
// keep smaller chunks so that the launch still fills the chip.
DecodePlan decode_plan(int32_t B, int32_t Hkv, int32_t max_kv_len, const muse_kv_cache* c) {
  DecodePlan d;
  if (c->kind == MUSE_KV_RING) {
    d.chunk_tokens = c->capacity >= kRingChunk ? kRingChunk : ((c->capacity + 31) / 32) * 32;
    d.max_chunks = (c->capacity + d.chunk_tokens - 1) / d.chunk_tokens;
  } else {
    d.chunk_tokens = kPagedChunkMax;
    const auto chunks = [&](int ct) { return (static_cast<int64_t>(max_kv_len) + ct - 1) / ct + 1; };
    while (d.chunk_tokens > kPagedChunkMin &&
           static_cast<int64_t>(B) * Hkv * chunks(d.chunk_tokens) < kPagedChunkTarget)
      d.chunk_tokens /= 2;
    d.max_chunks = static_cast<int>(chunks(d.chunk_tokens));
  }
  return d;
}

size_t decode_ws(const muse_attn_params* p, int32_t B, int32_t max_kv_len, const muse_kv_cache* c) {
  const DecodePlan d = decode_plan(B, p->num_kv_heads, max_kv_len, c);
  const int G = p->num_q_heads / p->num_kv_heads;
  size_t s = align256(static_cast<size_t>(B) * p->num_q_heads * p->head_dim * 4);
  s += align256(static_cast<size_t>(B) * p->num_kv_heads * p->head_dim * 4);
  s += align256(static_cast<size_t>(B) * p->num_kv_heads * d.max_chunks * G * (p->head_dim + 2) * 4);
  return s;
}

int32_t check_cache(const muse_attn_params* p, int32_t B, int32_t max_kv_len, const muse_kv_cache* c) {
  if (!c) return fail(MUSE_ERR_INVALID_ARG, "cache is NULL");
  if (!c->k || !c->v) return fail(MUSE_ERR_INVALID_ARG, "cache k/v is NULL");
  if (!aligned16(c->k) || !aligned16(c->v)) return fail(MUSE_ERR_INVALID_ARG, "cache k/v not 16-byte aligned");
  if (c->kind == MUSE_KV_RING) {
    if (p->sliding_window <= 0) return fail(MUSE_ERR_INVALID_ARG, "a ring cache needs a local layer (window > 0)");
    if (c->capacity != p->sliding_window)
      return fail(MUSE_ERR_INVALID_ARG, "ring capacity %d must equal the window %d", c->capacity, p->sliding_window);
    if (c->capacity % 16 != 0) return fail(MUSE_ERR_UNSUPPORTED, "ring capacity must be a multiple of 16");
  } else if (c->kind == MUSE_KV_PAGED) {
    if (!c->block_table) return fail(MUSE_ERR_INVALID_ARG, "block_table is NULL");
    if (c->page_tokens <= 0 || c->page_tokens % 16 != 0)
      return fail(MUSE_ERR_UNSUPPORTED, "page_tokens must be a positive multiple of 16");
    if (c->max_pages_per_seq <= 0 || c->num_pages <= 0)
      return fail(MUSE_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be positive");
    if (static_cast<int64_t>(max_kv_len) > static_cast<int64_t>(c->max_pages_per_seq) * c->page_tokens)
      return fail(MUSE_ERR_INVALID_ARG, "max_kv_len %d exceeds block-table capacity %lld", max_kv_len,
                  static_cast<long long>(c->max_pages_per_seq) * c->page_tokens);
  } else {
    return fail(MUSE_ERR_INVALID_ARG, "unknown cache kind %d", c->kind);
  }
  if (c->dtype == MUSE_DTYPE_FP8_E4M3) {
    if (!c->k_scale || !c->v_scale) return fail(MUSE_ERR_INVALID_ARG, "an E4M3 cache needs k_scale and v_scale");
  } else if (c->dtype != MUSE_DTYPE_BF16) {
    return fail(MUSE_ERR_UNSUPPORTED, "cache dtype %d (bf16 or E4M3 codes only)", c->dtype);
  }
  (void)B;
  return MUSE_OK;
}

// {batch, token} strides of q, k, v, gate, out (elements): the caller's, or
// those of contiguous [B, T, H, D] tensors; checked.
int32_t layer_strides(const muse_attn_params* p, int32_t T, const int64_t* strides, int64_t* s) {
  const int D = p->head_dim, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  if (strides) {
    memcpy(s, strides, 10 * sizeof(int64_t));
  } else {
    const int64_t hs[5] = {static_cast<int64_t>(Hq) * D, static_cast<int64_t>(Hkv) * D,
                           static_cast<int64_t>(Hkv) * D, static_cast<int64_t>(Hq) * D,
                           static_cast<int64_t>(Hq) * D};
    for (int i = 0; i < 5; ++i) {
      s[2 * i + 1] = hs[i];
      s[2 * i] = hs[i] * T;
    }
  }
  const int heads_of[5] = {Hq, Hkv, Hkv, Hq, Hq};
  for (int i = 0; i < 5; ++i) {
    if (s[2 * i] % 8 || s[2 * i + 1] % 8 || s[2 * i] < 0 || s[2 * i + 1] < 0)
      return fail(MUSE_ERR_INVALID_ARG, "strides must be non-negative multiples of 8 elements");
    if (s[2 * i + 1] < static_cast<int64_t>(heads_of[i]) * D)
      return fail(MUSE_ERR_INVALID_ARG, "token stride of tensor %d smaller than H * D", i);
  }
  return 0;
}

CacheView cache_view(const muse_kv_cache* c) {
  CacheView v{};
  v.kind = c->kind;
  v.capacity = c->capacity;
  v.max_pages = c->max_pages_per_seq;
  v.page_tokens = c->page_tokens;
  v.num_pages = c->num_pages;
  v.block_table = c->block_table;
  v.k = c->k;
  v.v = c->v;
  v.fp8 = c->dtype == MUSE_DTYPE_FP8_E4M3 ? 1 : 0;
  v.k_scale = c->k_scale;
  v.v_scale = c->v_scale;
  return v;
}

// The block's workspace: h as bf16 hi rows then lo rows [2R, hidden]; the
// projection of both halves in fp32 [2R, N]; the layer's inputs [R, N]
// (q, k, gate fp16, v bf16); o [R, Hq D] bf16; the o_proj output [R, hidden]
// fp32; the residual gate's coefficients; the GEMM scratch; then the
// layer's own workspace.
constexpr size_t kBlockGemmScratch = size_t(64) << 20;
// A hidden size the block kernels take: a positive multiple of 8 up to
// kBlockMaxHidden.
bool block_hidden_ok(int hidden) { return hidden > 0 && hidden % 8 == 0 && hidden <= kBlockMaxHidden; }
struct BlockWs {
  size_t h, proj, lay, o, a, coef, gemm, attn, total;
};
BlockWs block_ws_layout(const muse_attn_params* p, const muse_block_weights* w, int32_t B, int32_t T) {
  const size_t R = static_cast<size_t>(B) * T;
  const size_t D = p->head_dim, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  const size_t N = (2 * Hq + 2 * Hkv) * D;
  BlockWs l;
  l.h = 0;
  l.proj = l.h + align256(2 * R * w->hidden * 2);
  l.lay = l.proj + align256(2 * R * N * 4);
  l.o = l.lay + align256(R * N * 2);
  l.a = l.o + align256(R * Hq * D * 2);
  l.coef = l.a + align256(R * w->hidden * 4);
  l.gemm = l.coef + align256(static_cast<size_t>(w->hidden) * 8);
  l.attn = l.gemm + kBlockGemmScratch;
  l.total = l.attn + prefill_ws(p, B, T);
  return l;
}

// The decode step through the block: the same buffers for B one-token rows,
// then the decode workspace instead of the prefill one.
BlockWs block_decode_ws_layout(const muse_attn_params* p, const muse_block_weights* w, int32_t B,
                               int32_t max_kv_len, const muse_kv_cache* c) {
  BlockWs l = block_ws_layout(p, w, B, 1);
  l.total = l.attn + decode_ws(p, B, max_kv_len, c);
  return l;
}

}  // namespace

extern "C" {

int32_t muse_version(void) { return 105; }

const char* muse_last_error(void) { return g_err; }

int32_t muse_profile_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return fail(MUSE_ERR_INVALID_ARG, "pass both events or neither");
  g_prof_start = static_cast<hipEvent_t>(start);
  g_prof_stop = static_cast<hipEvent_t>(stop);
  return ok();
}

int32_t muse_layer_is_global(int32_t i, int32_t n_layers) {
  if (n_layers <= 0 || i < 0 || i >= n_layers) return -1;
  return ((n_layers - 1 - i) % 4) == 0 ? 1 : 0;
}

int32_t muse_rope_qknorm(const muse_attn_params* params, int32_t n_tokens, const void* q, int64_t q_stride_tok,
                         const void* k, int64_t k_stride_tok, const int32_t* positions, void* q_out, void* k_out,
                         int32_t out_dtype, void* stream) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (n_tokens < 0) return fail(MUSE_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (out_dtype != MUSE_DTYPE_BF16 && out_dtype != MUSE_DTYPE_F16 && out_dtype != MUSE_DTYPE_F32)
    return fail(MUSE_ERR_INVALID_ARG, "out_dtype %d unknown", out_dtype);
  if (!q && !k) return fail(MUSE_ERR_INVALID_ARG, "q and k are both NULL");
  if ((q && !q_out) || (k && !k_out)) return fail(MUSE_ERR_INVALID_ARG, "output pointer missing");
  const int D = params->head_dim;
  if (q && q_stride_tok < static_cast<int64_t>(params->num_q_heads) * D)
    return fail(MUSE_ERR_INVALID_ARG, "q_stride_tok smaller than Hq * D");
  if (k && k_stride_tok < static_cast<int64_t>(params->num_kv_heads) * D)
    return fail(MUSE_ERR_INVALID_ARG, "k_stride_tok smaller than Hkv * D");
  if (n_tokens == 0) return ok();
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  RopeQkArgs a{};
  a.positions = positions;
  a.eps = params->qk_norm_eps;
  a.log2_theta = log2_theta(params);
  a.use_rope = params->rope_theta > 0.f ? 1 : 0;
  if (q) {
    a.x = static_cast<const uint16_t*>(q);
    a.stride_tok = q_stride_tok;
    a.heads = params->num_q_heads;
    a.n_rows = static_cast<int64_t>(n_tokens) * params->num_q_heads;
    a.scale = params->qk_scale;
    a.out = q_out;
    hipError_t e = launch_rope_qknorm(D, out_dtype, a, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "rope_qknorm launch: %s", hipGetErrorString(e));
  }
  if (k) {
    a.x = static_cast<const uint16_t*>(k);
    a.stride_tok = k_stride_tok;
    a.heads = params->num_kv_heads;
    a.n_rows = static_cast<int64_t>(n_tokens) * params->num_kv_heads;
    a.scale = 1.0f;
    a.out = k_out;
    hipError_t e = launch_rope_qknorm(D, out_dtype, a, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "rope_qknorm launch: %s", hipGetErrorString(e));
  }
  return ok();
}

size_t muse_attn_prefill_workspace_size(const muse_attn_params* params, int32_t B, int32_t T) {
  if (check_params(params) || B < 0 || T < 0) return 0;
  return prefill_ws(params, B, T);
}

}  // extern "C"

namespace {
// The whole-sequence prefill; in_f16: q, k and gate arrive in fp16 (the
// decoder block's projections), else bf16 (the public entry point).
int32_t prefill_call(const muse_attn_params* params, int32_t B, int32_t T, const void* q, const void* k,
                     const void* v, const void* gate, const int64_t* strides, const int32_t* positions, void* out,
                     void* workspace, size_t ws_bytes, void* stream, int in_f16) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (B < 0 || T < 0) return fail(MUSE_ERR_INVALID_ARG, "B and T must be >= 0");
  if (B == 0 || T == 0) return ok();
  if (!q || !k || !v || !gate || !out) return fail(MUSE_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out))
    return fail(MUSE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const int D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  int64_t s[10];
  rc = layer_strides(params, T, strides, s);
  if (rc) return rc;
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const size_t need = prefill_ws(params, B, T);
  if (ws_bytes < need)
    return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n_tiles = prefill_tiles(T);
  {
    // launch-size limits, checked before any launch
    const int bq = prefill_rows_per_block(D, Hq / Hkv) / (Hq / Hkv);
    const int qgroup = prefill_qblock_group();
    const int64_t nq = (static_cast<int64_t>(T) + bq - 1) / bq;
    const int64_t nq_pad = ((nq + qgroup - 1) / qgroup) * qgroup;
    if (nq_pad * B * Hkv > 0x7fffffffLL || n_tiles * Hkv > 0x7fffffffLL || B > 65535)
      return fail(MUSE_ERR_UNSUPPORTED, "problem too large for one launch");
  }
  const PrefillWs wl = prefill_ws_layout(params, B, T);
  u32x4* tiles = static_cast<u32x4*>(workspace);
  float2* rope = wl.rope_bytes ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + wl.tile_bytes) : nullptr;
  hipError_t e;
  if (rope) {
    RopeTableArgs ra{};
    ra.positions = positions;
    ra.T = T;
    ra.n_rows = positions ? static_cast<int64_t>(B) * T : T;
    ra.log2_theta = log2_theta(params);
    ra.table = rope;
    e = launch_rope_table(D, ra, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "rope table launch: %s", hipGetErrorString(e));
  }

  KvPrepArgs kp{};
  kp.k = static_cast<const uint16_t*>(k);
  kp.v = static_cast<const uint16_t*>(v);
  kp.k_sb = s[2];
  kp.k_st = s[3];
  kp.v_sb = s[4];
  kp.v_st = s[5];
  kp.rope = rope;
  kp.rope_batched = positions ? 1 : 0;
  kp.T = T;
  kp.Hkv = Hkv;
  kp.n_tiles = static_cast<int>(n_tiles);
  kp.eps = params->qk_norm_eps;
  kp.tiles = tiles;
  kp.k_f16 = in_f16;
  e = launch_kv_prep(D, B, kp, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "kv_prep launch: %s", hipGetErrorString(e));

  const int G = Hq / Hkv;
  const int rows = prefill_rows_per_block(D, G);
  const int bq = rows / G;
  const int qgroup = prefill_qblock_group();
  PrefillArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.gate = static_cast<const uint16_t*>(gate);
  pa.in_f16 = in_f16;
  pa.out = static_cast<uint16_t*>(out);
  pa.tiles = tiles;
  pa.q_sb = s[0];
  pa.q_st = s[1];
  pa.g_sb = s[6];
  pa.g_st = s[7];
  pa.o_sb = s[8];
  pa.o_st = s[9];
  pa.rope = rope;
  pa.rope_batched = positions ? 1 : 0;
  pa.T = T;
  pa.Hkv = Hkv;
  pa.W = params->sliding_window;
  pa.n_tiles = static_cast<int>(n_tiles);
  pa.n_qblocks = (T + bq - 1) / bq;
  pa.n_qblocks_pad = ((pa.n_qblocks + qgroup - 1) / qgroup) * qgroup;
  pa.batch_heads = B * Hkv;
  pa.qscale = q_logit_scale(params);
  pa.qk_eps = params->qk_norm_eps;
  pa.out_norm = params->out_norm;
  pa.out_eps = params->out_norm_eps;
  if (g_prof_start) {
    e = hipEventRecord(g_prof_start, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  e = launch_prefill(D, G, pa, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  if (g_prof_stop) {
    e = hipEventRecord(g_prof_stop, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  return ok();
}
}  // namespace

extern "C" {

int32_t muse_attn_prefill(const muse_attn_params* params, int32_t B, int32_t T, const void* q, const void* k,
                          const void* v, const void* gate, const int64_t* strides, const int32_t* positions,
                          void* out, void* workspace, size_t ws_bytes, void* stream) {
  return prefill_call(params, B, T, q, k, v, gate, strides, positions, out, workspace, ws_bytes, stream, 0);
}

size_t muse_attn_prefill_chunk_workspace_size(const muse_attn_params* params, int32_t B, int32_t T,
                                              int32_t max_start) {
  if (check_params(params) || B < 0 || T < 0 || max_start < 0) return 0;
  return chunk_ws_layout(params, B, T, max_start).total;
}

}  // extern "C"

namespace {
// Chunked prefill and the drafter's non-causal block: the same three steps
// (tile image of history + chunk, attention, and for the chunk the cache
// write), with the causal mask or the bidirectional window.
int32_t chunk_call(const muse_attn_params* params, int32_t B, int32_t T, const void* q, const void* k,
                   const void* v, const void* gate, const int64_t* strides, const int32_t* start,
                   int32_t max_start, const muse_kv_cache* cache, void* out, void* workspace, size_t ws_bytes,
                   void* stream, bool noncausal) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (B < 0 || T < 0) return fail(MUSE_ERR_INVALID_ARG, "B and T must be >= 0");
  if (max_start < 0) return fail(MUSE_ERR_INVALID_ARG, "max_start must be >= 0");
  if (static_cast<int64_t>(max_start) + T > 0x7fffffffLL)
    return fail(MUSE_ERR_UNSUPPORTED, "max_start + T exceeds the 32-bit position range");
  // a chunk is written after positions up to max_start + T - 1; a block only
  // reads positions below max_start
  rc = check_cache(params, B, std::max(1, noncausal ? max_start : max_start + T), cache);
  if (rc) return rc;
  if (B == 0 || T == 0) return ok();
  if (!q || !k || !v || !gate || !out || !start) return fail(MUSE_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out))
    return fail(MUSE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const int D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  int64_t s[10];
  rc = layer_strides(params, T, strides, s);
  if (rc) return rc;
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const PrefillWs wl = chunk_ws_layout(params, B, T, max_start);
  if (ws_bytes < wl.total)
    return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, wl.total);
  const int64_t n_tiles = chunk_tiles(params, T, max_start);
  const int G = Hq / Hkv;
  const int rows = prefill_rows_per_block(D, G);
  const int bq = rows / G;
  const int qgroup = prefill_qblock_group();
  const int64_t nq = (static_cast<int64_t>(T) + bq - 1) / bq;
  const int64_t nq_pad = ((nq + qgroup - 1) / qgroup) * qgroup;
  if (nq_pad * B * Hkv > 0x7fffffffLL || n_tiles * Hkv > 0x7fffffffLL || B > 65535)
    return fail(MUSE_ERR_UNSUPPORTED, "problem too large for one launch");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  u32x4* tiles = static_cast<u32x4*>(workspace);
  float2* rope = wl.rope_bytes ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + wl.tile_bytes) : nullptr;
  const CacheView cv = cache_view(cache);
  hipError_t e;
  if (rope) {
    RopeTableArgs ra{};
    ra.start = start;
    ra.max_start = max_start;
    ra.T = T;
    ra.n_rows = static_cast<int64_t>(B) * T;
    ra.log2_theta = log2_theta(params);
    ra.table = rope;
    e = launch_rope_table(D, ra, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "rope table launch: %s", hipGetErrorString(e));
  }

  // 1. tile image: cached history (as stored) and the chunk's own keys/values
  KvPrepArgs kp{};
  kp.k = static_cast<const uint16_t*>(k);
  kp.v = static_cast<const uint16_t*>(v);
  kp.k_sb = s[2];
  kp.k_st = s[3];
  kp.v_sb = s[4];
  kp.v_st = s[5];
  kp.rope = rope;
  kp.rope_batched = 1;
  kp.T = T;
  kp.Hkv = Hkv;
  kp.n_tiles = static_cast<int>(n_tiles);
  kp.eps = params->qk_norm_eps;
  kp.tiles = tiles;
  kp.start = start;
  kp.max_start = max_start;
  kp.W = params->sliding_window;
  kp.cache = cv;
  char* ws_parts = static_cast<char*>(workspace) + wl.tile_bytes + wl.rope_bytes;
  kp.tile_ms = reinterpret_cast<float*>(ws_parts + wl.part_o_bytes + wl.part_l_bytes);
  e = launch_kv_prep(D, B, kp, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "kv_prep launch: %s", hipGetErrorString(e));

  // 2. attention over the tile image
  PrefillArgs pa{};
  pa.q = static_cast<const uint16_t*>(q);
  pa.gate = static_cast<const uint16_t*>(gate);
  pa.out = static_cast<uint16_t*>(out);
  pa.tiles = tiles;
  pa.q_sb = s[0];
  pa.q_st = s[1];
  pa.g_sb = s[6];
  pa.g_st = s[7];
  pa.o_sb = s[8];
  pa.o_st = s[9];
  pa.rope = rope;
  pa.rope_batched = 1;
  pa.T = T;
  pa.Hkv = Hkv;
  pa.W = params->sliding_window;
  pa.n_tiles = static_cast<int>(n_tiles);
  pa.n_qblocks = static_cast<int>(nq);
  pa.n_qblocks_pad = static_cast<int>(nq_pad);
  pa.batch_heads = B * Hkv;
  pa.qscale = q_logit_scale(params);
  pa.qk_eps = params->qk_norm_eps;
  pa.out_norm = params->out_norm;
  pa.out_eps = params->out_norm_eps;
  pa.start = start;
  pa.max_start = max_start;
  pa.noncausal = noncausal ? 1 : 0;
  pa.nsplit = wl.nsplit;
  pa.tile_ms = kp.tile_ms;
  pa.qbound = static_cast<float>(static_cast<double>(pa.qscale) * D * (1.0 + 1.0 / 256));
  pa.part_o = wl.nsplit > 1 ? reinterpret_cast<float*>(ws_parts) : nullptr;
  pa.part_l = wl.nsplit > 1 ? reinterpret_cast<float*>(ws_parts + wl.part_o_bytes) : nullptr;
  if (g_prof_start) {
    e = hipEventRecord(g_prof_start, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  e = launch_prefill(D, G, pa, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  if (wl.nsplit > 1) {
    PrefillCombineArgs pc{};
    pc.part_o = pa.part_o;
    pc.part_l = pa.part_l;
    pc.nsplit = wl.nsplit;
    pc.gate = pa.gate;
    pc.out = pa.out;
    pc.g_sb = s[6];
    pc.g_st = s[7];
    pc.o_sb = s[8];
    pc.o_st = s[9];
    pc.B = B;
    pc.T = T;
    pc.Hq = Hq;
    pc.out_norm = params->out_norm;
    pc.out_eps = params->out_norm_eps;
    pc.start = start;
    pc.max_start = max_start;
    e = launch_prefill_combine(D, pc, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "prefill combine launch: %s", hipGetErrorString(e));
  }
  if (g_prof_stop) {
    e = hipEventRecord(g_prof_stop, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }

  if (noncausal) return ok();  // a drafter's block is not kept in the cache

  // 3. the chunk's keys and values into the cache (after every read of it)
  ChunkAppendArgs ca{};
  ca.k = kp.k;
  ca.v = kp.v;
  ca.k_sb = s[2];
  ca.k_st = s[3];
  ca.v_sb = s[4];
  ca.v_st = s[5];
  ca.rope = rope;
  ca.start = start;
  ca.max_start = max_start;
  ca.T = T;
  ca.Hkv = Hkv;
  ca.W = params->sliding_window;
  ca.eps = params->qk_norm_eps;
  ca.cache = cv;
  e = launch_chunk_append(D, B, ca, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "chunk append launch: %s", hipGetErrorString(e));
  return ok();
}
// The drafter's block as a few-token decode (blocks with T <= 64 and
// T * G <= 128 columns per KV head): a split pass over each sequence's
// cached context that also forms the queries and the block's own-key term,
// and a combine of the partials with the epilogue.  The cache is read as
// stored, once per 64 columns.  Workspace: one partial row of D + 4 floats
// per (sequence, KV head, column group, split workgroup, column).
size_t draft_ws(const muse_attn_params* p, int32_t B, int32_t T, int32_t max_start) {
  const int D = p->head_dim, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  const DraftPlan pl = draft_plan(B, Hkv, Hq / Hkv, T, p->sliding_window, max_start);
  return align256(static_cast<size_t>(B) * Hkv * pl.n_cgroups * pl.n_wg * kDraftGroupCols * (D + 4) * 4);
}

int32_t draft_call(const muse_attn_params* params, int32_t B, int32_t T, const void* q, const void* k,
                   const void* v, const void* gate, const int64_t* strides, const int32_t* start, int32_t max_start,
                   const muse_kv_cache* cache, void* out, void* workspace, size_t ws_bytes, void* stream) {
  if (B < 0 || T < 0) return fail(MUSE_ERR_INVALID_ARG, "B and T must be >= 0");
  if (max_start < 0) return fail(MUSE_ERR_INVALID_ARG, "max_start must be >= 0");
  if (static_cast<int64_t>(max_start) + T > 0x7fffffffLL)
    return fail(MUSE_ERR_UNSUPPORTED, "max_start + T exceeds the 32-bit position range");
  int32_t rc = check_cache(params, B, std::max(1, max_start), cache);
  if (rc) return rc;
  if (B == 0 || T == 0) return ok();
  if (!q || !k || !v || !gate || !out || !start) return fail(MUSE_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gate) || !aligned16(out))
    return fail(MUSE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const int D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  int64_t s[10];
  rc = layer_strides(params, T, strides, s);
  if (rc) return rc;
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const size_t need = draft_ws(params, B, T, max_start);
  if (ws_bytes < need) return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  const DraftPlan pl = draft_plan(B, Hkv, Hq / Hkv, T, params->sliding_window, max_start);
  if (static_cast<int64_t>(B) * Hkv * pl.n_cgroups * pl.n_wg > 0x7fffffffLL ||
      static_cast<int64_t>(B) * T * ((Hq + 3) / 4) > 0x7fffffffLL)
    return fail(MUSE_ERR_UNSUPPORTED, "problem too large for one launch");
  rc = check_device();
  if (rc) return rc;
  DraftArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.gate = static_cast<const uint16_t*>(gate);
  a.q_sb = s[0];
  a.q_st = s[1];
  a.k_sb = s[2];
  a.k_st = s[3];
  a.v_sb = s[4];
  a.v_st = s[5];
  a.g_sb = s[6];
  a.g_st = s[7];
  a.o_sb = s[8];
  a.o_st = s[9];
  a.out = static_cast<uint16_t*>(out);
  a.start = start;
  a.max_start = max_start;
  a.B = B;
  a.T = T;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.W = params->sliding_window;
  a.qscale = q_logit_scale(params);
  a.qk_eps = params->qk_norm_eps;
  a.out_eps = params->out_norm_eps;
  a.out_norm = params->out_norm;
  a.log2_theta = log2_theta(params);
  a.use_rope = params->rope_theta > 0.f ? 1 : 0;
  a.cache = cache_view(cache);
  a.chunk_tokens = pl.chunk_tokens;
  a.n_cgroups = pl.n_cgroups;
  a.n_wg = pl.n_wg;
  a.part = static_cast<float*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (g_prof_start) {
    e = hipEventRecord(g_prof_start, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  e = launch_draft(D, a, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "draft launch: %s", hipGetErrorString(e));
  if (g_prof_stop) {
    e = hipEventRecord(g_prof_stop, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  return ok();
}

int32_t decode_call(const muse_attn_params* params, int32_t B, const void* q_new, int64_t q_sb, const void* k_new,
                    const void* v_new, int64_t kv_sb, const void* gate, int64_t g_sb, const int32_t* kv_len,
                    int32_t max_kv_len, const muse_kv_cache* cache, void* out, void* workspace, size_t ws_bytes,
                    void* stream, int in_f16 = 0);
}  // namespace

extern "C" {

int32_t muse_attn_prefill_chunk(const muse_attn_params* params, int32_t B, int32_t T, const void* q,
                                const void* k, const void* v, const void* gate, const int64_t* strides,
                                const int32_t* start, int32_t max_start, const muse_kv_cache* cache, void* out,
                                void* workspace, size_t ws_bytes, void* stream) {
  return chunk_call(params, B, T, q, k, v, gate, strides, start, max_start, cache, out, workspace, ws_bytes, stream,
                    false);
}

size_t muse_attn_draft_block_workspace_size(const muse_attn_params* params, int32_t B, int32_t T,
                                            int32_t max_start) {
  if (check_params(params) || B < 0 || T < 0 || max_start < 0) return 0;
  if (draft_split_fits(T, params->num_q_heads / params->num_kv_heads)) return draft_ws(params, B, T, max_start);
  return muse_attn_prefill_chunk_workspace_size(params, B, T, max_start);
}

int32_t muse_attn_draft_block(const muse_attn_params* params, int32_t B, int32_t T, const void* q, const void* k,
                              const void* v, const void* gate, const int64_t* strides, const int32_t* start,
                              int32_t max_start, const muse_kv_cache* cache, void* out, void* workspace,
                              size_t ws_bytes, void* stream) {
  const int32_t rc = check_params(params);
  if (rc) return rc;
  if (draft_split_fits(T, params->num_q_heads / params->num_kv_heads))
    return draft_call(params, B, T, q, k, v, gate, strides, start, max_start, cache, out, workspace, ws_bytes,
                      stream);
  return chunk_call(params, B, T, q, k, v, gate, strides, start, max_start, cache, out, workspace, ws_bytes, stream,
                    true);
}

size_t muse_attn_decode_workspace_size(const muse_attn_params* params, int32_t B, int32_t max_kv_len,
                                       const muse_kv_cache* cache) {
  if (check_params(params) || B < 0 || max_kv_len < 1 || !cache) return 0;
  if (cache->kind == MUSE_KV_RING && cache->capacity <= 0) return 0;
  return decode_ws(params, B, max_kv_len, cache);
}

int32_t muse_attn_decode(const muse_attn_params* params, int32_t B, const void* q_new, const void* k_new,
                         const void* v_new, const void* gate, const int32_t* kv_len, int32_t max_kv_len,
                         const muse_kv_cache* cache, void* out, void* workspace, size_t ws_bytes, void* stream) {
  const int32_t rc = check_params(params);
  if (rc) return rc;
  const int64_t qs = static_cast<int64_t>(params->num_q_heads) * params->head_dim;
  const int64_t ks = static_cast<int64_t>(params->num_kv_heads) * params->head_dim;
  return decode_call(params, B, q_new, qs, k_new, v_new, ks, gate, qs, kv_len, max_kv_len, cache, out, workspace,
                     ws_bytes, stream);
}

}  // extern "C"

namespace {
// One decode step; q_new and gate rows of each sequence are q_sb and g_sb
// elements apart, k_new and v_new rows kv_sb (contiguous for the public
// entry point, the projection rows for the decoder block).
int32_t decode_call(const muse_attn_params* params, int32_t B, const void* q_new, int64_t q_sb, const void* k_new,
                    const void* v_new, int64_t kv_sb, const void* gate, int64_t g_sb, const int32_t* kv_len,
                    int32_t max_kv_len, const muse_kv_cache* cache, void* out, void* workspace, size_t ws_bytes,
                    void* stream, int in_f16) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (B < 0) return fail(MUSE_ERR_INVALID_ARG, "B must be >= 0");
  if (max_kv_len < 1) return fail(MUSE_ERR_INVALID_ARG, "max_kv_len must be >= 1");
  rc = check_cache(params, B, max_kv_len, cache);
  if (rc) return rc;
  if (B == 0) return ok();
  if (!q_new || !k_new || !v_new || !gate || !kv_len || !out)
    return fail(MUSE_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(gate) || !aligned16(out))
    return fail(MUSE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const size_t need = decode_ws(params, B, max_kv_len, cache);
  if (ws_bytes < need) return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  rc = check_device();
  if (rc) return rc;
  const DecodePlan plan = decode_plan(B, params->num_kv_heads, max_kv_len, cache);
  const int D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  if (static_cast<int64_t>(B) * Hkv * plan.max_chunks > 0x7fffffffLL)
    return fail(MUSE_ERR_UNSUPPORTED, "problem too large for one launch");
  DecodeArgs a{};
  a.in_f16 = in_f16;
  a.q_new = static_cast<const uint16_t*>(q_new);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.gate = static_cast<const uint16_t*>(gate);
  a.q_sb = q_sb;
  a.kv_sb = kv_sb;
  a.g_sb = g_sb;
  a.kv_len = kv_len;
  a.out = static_cast<uint16_t*>(out);
  a.kc = static_cast<uint16_t*>(cache->k);
  a.vc = static_cast<uint16_t*>(cache->v);
  a.fp8 = cache->dtype == MUSE_DTYPE_FP8_E4M3 ? 1 : 0;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_table = cache->block_table;
  a.kind = cache->kind;
  a.capacity = cache->capacity;
  a.max_pages = cache->max_pages_per_seq;
  a.page_tokens = cache->page_tokens;
  a.num_pages = cache->num_pages;
  a.B = B;
  a.Hkv = Hkv;
  a.W = params->sliding_window;
  a.max_kv_len = max_kv_len;
  a.chunk_tokens = plan.chunk_tokens;
  a.max_chunks = plan.max_chunks;
  a.qscale = q_logit_scale(params);
  a.qk_eps = params->qk_norm_eps;
  a.out_eps = params->out_norm_eps;
  a.log2_theta = log2_theta(params);
  a.use_rope = params->rope_theta > 0.f ? 1 : 0;
  a.out_norm = params->out_norm;
  char* ws = static_cast<char*>(workspace);
  a.qhat = reinterpret_cast<float*>(ws);
  ws += align256(static_cast<size_t>(B) * Hq * D * 4);
  a.khat = reinterpret_cast<float*>(ws);
  ws += align256(static_cast<size_t>(B) * Hkv * D * 4);
  a.part = reinterpret_cast<float*>(ws);
  hipError_t e = launch_decode(D, Hq / Hkv, a, static_cast<hipStream_t>(stream), g_prof_start, g_prof_stop);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

// The device address of `scratch` on the current device, fetched once per
// device with that device current.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MUSE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(MUSE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUSE_OK;
}
}  // namespace

extern "C" {

int32_t muse_attn_decode_noalloc(const muse_attn_params* params, int32_t B, const void* q_new, const void* k_new,
                                 const void* v_new, const void* gate, const int32_t* kv_len, int32_t max_kv_len,
                                 const muse_kv_cache* cache, void* out, void* stream) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (B < 0) return fail(MUSE_ERR_INVALID_ARG, "B must be >= 0");
  if (max_kv_len < 1) return fail(MUSE_ERR_INVALID_ARG, "max_kv_len must be >= 1");
  rc = check_cache(params, B, max_kv_len, cache);
  if (rc) return rc;
  if (B == 0) return ok();
  const size_t need = decode_ws(params, B, max_kv_len, cache);
  if (need > MUSE_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(MUSE_ERR_WORKSPACE,
                "muse_attn_decode_noalloc: this call needs %zu bytes of scratch, above its fixed %zu; "
                "use muse_attn_decode with a workspace",
                need, static_cast<size_t>(MUSE_DECODE_NOALLOC_SCRATCH_BYTES));
  rc = check_device();
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  const int64_t qs = static_cast<int64_t>(params->num_q_heads) * params->head_dim;
  const int64_t ks = static_cast<int64_t>(params->num_kv_heads) * params->head_dim;
  return decode_call(params, B, q_new, qs, k_new, v_new, ks, gate, qs, kv_len, max_kv_len, cache, out, ws,
                     MUSE_DECODE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {
// The decoder block around the layer, before it: input norm (h as bf16 hi
// and lo rows), the q/k/v/gate projection of both halves (fp32), and their
// sum handed to the layer (q, k, gate fp16; v bf16) in `lay`.
int32_t block_front(const muse_attn_params* params, const muse_block_weights* w, int64_t R, const void* x,
                    const BlockWs& l, char* ws, hipStream_t st) {
  const int64_t D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  const int64_t N = (2 * Hq + 2 * Hkv) * D;
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + l.h);
  BlockNormArgs na{};
  na.x = static_cast<const uint16_t*>(x);
  na.w = static_cast<const uint16_t*>(w->in_norm);
  na.out = h;
  na.out_lo = h + R * w->hidden;
  na.rows = R;
  na.hidden = w->hidden;
  na.eps = 1e-5f;
  hipError_t e = launch_block_input_norm(na, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "input norm launch: %s", hipGetErrorString(e));
  char msg[256];
  float* proj = reinterpret_cast<float*>(ws + l.proj);
  if (block_gemm(2 * R, N, w->hidden, h, w->w_qkvg, proj, ws + l.gemm, kBlockGemmScratch, st, msg, sizeof(msg)))
    return fail(MUSE_ERR_HIP, "q/k/v/gate projection: %s", msg);
  BlockProjPrepArgs pp{};
  pp.proj = proj;
  pp.out = reinterpret_cast<uint16_t*>(ws + l.lay);
  pp.rows = R;
  pp.n = static_cast<int>(N);
  pp.q_end = static_cast<int>(Hq * D);
  pp.k_end = static_cast<int>((Hq + Hkv) * D);
  pp.v_end = static_cast<int>((Hq + 2 * Hkv) * D);
  e = launch_block_proj_prep(pp, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "projection prep launch: %s", hipGetErrorString(e));
  return MUSE_OK;
}

// After the layer: o_proj (fp32 out), then the post-attention norm and the
// residual (Glimmer's centered norm and add, or Spark's residual gate).
int32_t block_back(const muse_attn_params* params, const muse_block_weights* w, int64_t R, const void* x,
                   void* out, const BlockWs& l, char* ws, hipStream_t st) {
  const int64_t D = params->head_dim, Hq = params->num_q_heads;
  float* a = reinterpret_cast<float*>(ws + l.a);
  char msg[256];
  if (block_gemm(R, w->hidden, Hq * D, ws + l.o, w->w_o, a, ws + l.gemm, kBlockGemmScratch, st, msg, sizeof(msg)))
    return fail(MUSE_ERR_HIP, "o_proj: %s", msg);
  float2* coef = nullptr;
  hipError_t e;
  if (w->residual_gate) {
    coef = reinterpret_cast<float2*>(ws + l.coef);
    e = launch_block_gate_coef(w->residual_gate, coef, w->hidden, w->residual_gate_temperature, 1e-3f, st);
    if (e != hipSuccess) return fail(MUSE_ERR_HIP, "gate coefficient launch: %s", hipGetErrorString(e));
  }
  BlockResidualArgs ra{};
  ra.x = static_cast<const uint16_t*>(x);
  ra.branch = a;
  ra.post_norm = static_cast<const uint16_t*>(w->post_norm);
  ra.coef = reinterpret_cast<const float*>(coef);
  ra.out = static_cast<uint16_t*>(out);
  ra.rows = R;
  ra.hidden = w->hidden;
  ra.eps = 1e-8f;
  e = launch_block_residual(ra, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "residual launch: %s", hipGetErrorString(e));
  return MUSE_OK;
}
}  // namespace

extern "C" {

size_t muse_attn_block_prefill_workspace_size(const muse_attn_params* params, const muse_block_weights* weights,
                                              int32_t B, int32_t T) {
  if (check_params(params) || !weights || !block_hidden_ok(weights->hidden) || B < 0 || T < 0) return 0;
  return block_ws_layout(params, weights, B, T).total;
}

int32_t muse_attn_block_prefill(const muse_attn_params* params, const muse_block_weights* w, int32_t B, int32_t T,
                                const void* x, void* out, void* workspace, size_t ws_bytes, void* stream) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (!w) return fail(MUSE_ERR_INVALID_ARG, "weights is NULL");
  if (B < 0 || T < 0) return fail(MUSE_ERR_INVALID_ARG, "B and T must be >= 0");
  if (!block_hidden_ok(w->hidden))
    return fail(MUSE_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 8 up to %d", w->hidden,
                kBlockMaxHidden);
  if (!w->in_norm || !w->w_qkvg || !w->w_o) return fail(MUSE_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (w->residual_gate ? !(w->residual_gate_temperature > 0.f) : !w->post_norm)
    return fail(MUSE_ERR_INVALID_ARG, "a plain add needs post_norm; a residual gate a positive temperature");
  if (B == 0 || T == 0) return ok();
  if (!x || !out) return fail(MUSE_ERR_INVALID_ARG, "x or out is NULL");
  const void* ptrs[] = {x, out, w->in_norm, w->w_qkvg, w->w_o, w->post_norm, w->residual_gate};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MUSE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const BlockWs l = block_ws_layout(params, w, B, T);
  if (ws_bytes < l.total) return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, l.total);
  if (static_cast<int64_t>(B) * T > 0x7fffffffLL) return fail(MUSE_ERR_UNSUPPORTED, "too many rows for one launch");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t R = static_cast<int64_t>(B) * T;
  const int64_t D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  const int64_t N = (2 * Hq + 2 * Hkv) * D;
  rc = block_front(params, w, R, x, l, ws, st);
  if (rc) return rc;
  // the layer on strided views of its inputs: q, k, v, gate columns
  const uint16_t* lay = reinterpret_cast<const uint16_t*>(ws + l.lay);
  const int64_t strides[10] = {T * N, N, T * N, N, T * N, N, T * N, N, T * Hq * D, Hq * D};
  rc = prefill_call(params, B, T, lay, lay + Hq * D, lay + (Hq + Hkv) * D, lay + (Hq + 2 * Hkv) * D, strides,
                    nullptr, ws + l.o, ws + l.attn, l.total - l.attn, stream, 1);
  if (rc) return rc;
  rc = block_back(params, w, R, x, out, l, ws, st);
  if (rc) return rc;
  return ok();
}

int32_t muse_attn_block_tune(const muse_attn_params* params, const muse_block_weights* w, int32_t rows,
                             void* workspace, size_t ws_bytes, void* stream) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (!w) return fail(MUSE_ERR_INVALID_ARG, "weights is NULL");
  if (rows <= 0) return fail(MUSE_ERR_INVALID_ARG, "rows must be > 0");
  if (!block_hidden_ok(w->hidden))
    return fail(MUSE_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 8 up to %d", w->hidden,
                kBlockMaxHidden);
  if (!w->w_qkvg || !w->w_o) return fail(MUSE_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (!aligned16(w->w_qkvg) || !aligned16(w->w_o)) return fail(MUSE_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const BlockWs l = block_ws_layout(params, w, 1, rows);
  if (ws_bytes < l.total) return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, l.total);
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  const int64_t N = (2 * Hq + 2 * Hkv) * D;
  // zero activations (h's two halves, o): the timed runs read defined values
  hipError_t e = hipMemsetAsync(ws + l.h, 0, l.proj - l.h, st);
  if (e == hipSuccess) e = hipMemsetAsync(ws + l.o, 0, l.a - l.o, st);
  if (e != hipSuccess) return fail(MUSE_ERR_HIP, "hipMemsetAsync: %s", hipGetErrorString(e));
  char msg[256];
  if (block_gemm(2 * static_cast<int64_t>(rows), N, w->hidden, ws + l.h, w->w_qkvg,
                 reinterpret_cast<float*>(ws + l.proj), ws + l.gemm, kBlockGemmScratch, st, msg, sizeof(msg), true))
    return fail(MUSE_ERR_HIP, "q/k/v/gate projection tuning: %s", msg);
  if (block_gemm(rows, w->hidden, Hq * D, ws + l.o, w->w_o, reinterpret_cast<float*>(ws + l.a), ws + l.gemm,
                 kBlockGemmScratch, st, msg, sizeof(msg), true))
    return fail(MUSE_ERR_HIP, "o_proj tuning: %s", msg);
  return ok();
}

size_t muse_attn_block_decode_workspace_size(const muse_attn_params* params, const muse_block_weights* weights,
                                             int32_t B, int32_t max_kv_len, const muse_kv_cache* cache) {
  if (check_params(params) || !weights || !block_hidden_ok(weights->hidden) || !cache || B < 0 || max_kv_len < 1)
    return 0;
  return block_decode_ws_layout(params, weights, B, max_kv_len, cache).total;
}

int32_t muse_attn_block_decode(const muse_attn_params* params, const muse_block_weights* w, int32_t B,
                               const void* x, const int32_t* kv_len, int32_t max_kv_len, const muse_kv_cache* cache,
                               void* out, void* workspace, size_t ws_bytes, void* stream) {
  int32_t rc = check_params(params);
  if (rc) return rc;
  if (!w) return fail(MUSE_ERR_INVALID_ARG, "weights is NULL");
  if (B < 0) return fail(MUSE_ERR_INVALID_ARG, "B must be >= 0");
  if (max_kv_len < 1) return fail(MUSE_ERR_INVALID_ARG, "max_kv_len must be >= 1");
  if (!block_hidden_ok(w->hidden))
    return fail(MUSE_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 8 up to %d", w->hidden,
                kBlockMaxHidden);
  if (!w->in_norm || !w->w_qkvg || !w->w_o) return fail(MUSE_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (w->residual_gate ? !(w->residual_gate_temperature > 0.f) : !w->post_norm)
    return fail(MUSE_ERR_INVALID_ARG, "a plain add needs post_norm; a residual gate a positive temperature");
  rc = check_cache(params, B, max_kv_len, cache);
  if (rc) return rc;
  if (B == 0) return ok();
  if (!x || !out || !kv_len) return fail(MUSE_ERR_INVALID_ARG, "x, out or kv_len is NULL");
  const void* ptrs[] = {x, out, w->in_norm, w->w_qkvg, w->w_o, w->post_norm, w->residual_gate};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MUSE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(MUSE_ERR_WORKSPACE, "workspace missing or misaligned");
  const BlockWs l = block_decode_ws_layout(params, w, B, max_kv_len, cache);
  if (ws_bytes < l.total) return fail(MUSE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, l.total);
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t D = params->head_dim, Hq = params->num_q_heads, Hkv = params->num_kv_heads;
  const int64_t N = (2 * Hq + 2 * Hkv) * D;
  rc = block_front(params, w, B, x, l, ws, st);
  if (rc) return rc;
  // the layer's decode step reads q, k, v and the gate straight from the rows of its inputs
  const uint16_t* lay = reinterpret_cast<const uint16_t*>(ws + l.lay);
  rc = decode_call(params, B, lay, N, lay + Hq * D, lay + (Hq + Hkv) * D, N, lay + (Hq + 2 * Hkv) * D, N, kv_len,
                   max_kv_len, cache, ws + l.o, ws + l.attn, l.total - l.attn, stream, 1);
  if (rc) return rc;
  rc = block_back(params, w, B, x, out, l, ws, st);
  if (rc) return rc;
  return ok();
}

}  // extern "C"
