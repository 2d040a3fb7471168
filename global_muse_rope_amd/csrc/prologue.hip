// Prologue kernels: weightless QK-norm, query multiplier and RoPE.
//
// Muse Spark Open deep dive, section 3.2 (steps 2-4: per-head RMS norm with
// eps inside the square root, multiplier on q only) and section 3.4 (RoPE on
// local layers, dimension j paired with j + D/2, angle p * theta^(-2j/D)).
#include "kernels.h"

namespace muse {

// ---------------------------------------------------------------------------
// Standalone prologue: one (token, head) row per D/2 lanes, one RoPE pair
// (j, j + D/2) per lane.
// ---------------------------------------------------------------------------
template <int D, int OUT>
__global__ __launch_bounds__(256) void rope_qknorm_kernel(RopeQkArgs a) {
  constexpr int LPR = D / 2;  // lanes per row
  const int64_t gtid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = gtid / LPR;
  const int j = static_cast<int>(gtid % LPR);
  const bool valid = row < a.n_rows;
  const int64_t t = valid ? row / a.heads : 0;
  const int h = valid ? static_cast<int>(row % a.heads) : 0;
  float x0 = 0.f, x1 = 0.f;
  if (valid) {
    const uint16_t* p = a.x + t * a.stride_tok + static_cast<int64_t>(h) * D;
    x0 = bf16_bits_to_f32(p[j]);
    x1 = bf16_bits_to_f32(p[j + D / 2]);
  }
  const float ss = group_sum<LPR>(x0 * x0 + x1 * x1);
  const float r = a.scale / sqrtf(ss * (1.0f / D) + a.eps);
  x0 *= r;
  x1 *= r;
  if (a.use_rope) {
    const int pos = a.positions ? a.positions[t] : static_cast<int>(t);
    float s, c;
    rope_sincos(pos, j, D, a.log2_theta, &s, &c);
    const float y0 = x0 * c - x1 * s;
    const float y1 = x1 * c + x0 * s;
    x0 = y0;
    x1 = y1;
  }
  if (!valid) return;
  const int64_t o = row * D;
  if (OUT == MUSE_DTYPE_F32) {
    float* out = static_cast<float*>(a.out);
    out[o + j] = x0;
    out[o + j + D / 2] = x1;
  } else if (OUT == MUSE_DTYPE_F16) {
    half_t* out = static_cast<half_t*>(a.out);
    out[o + j] = static_cast<half_t>(x0);
    out[o + j + D / 2] = static_cast<half_t>(x1);
  } else {
    uint16_t* out = static_cast<uint16_t*>(a.out);
    out[o + j] = f32_to_bf16_bits(x0);
    out[o + j + D / 2] = f32_to_bf16_bits(x1);
  }
}

// ---------------------------------------------------------------------------
// RoPE table for a prefill call: one (cos, sin) pair per (position row, j).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableArgs a) {
  const int64_t gt = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gt >= a.n_rows * (D / 2)) return;
  const int64_t row = gt / (D / 2);
  const int j = static_cast<int>(gt % (D / 2));
  int pos;
  if (a.start) {
    const int st = a.start[row / a.T];
    pos = (chunk_start_ok(st, a.max_start) ? st : 0) + static_cast<int>(row % a.T);
  } else {
    pos = a.positions ? a.positions[row] : static_cast<int>(row % a.T);
  }
  float s, c;
  rope_sincos(pos, j, D, a.log2_theta, &s, &c);
  a.table[gt] = make_float2(c, s);
}

// ---------------------------------------------------------------------------
// Where a cached position lives: element offsets of its key row and of its
// value column (dimension 0; dimension d adds d * value stride), the scale
// index of an E4M3 cache, and whether its page is present.
// ---------------------------------------------------------------------------
struct CacheLoc {
  int64_t k, v;
  int si;
  bool ok;
};

__device__ __forceinline__ CacheLoc cache_loc(const CacheView& c, int b, int hk, int Hkv, int D, int pos) {
  CacheLoc l;
  if (c.kind == MUSE_KV_RING) {
    const int64_t bh = static_cast<int64_t>(b) * Hkv + hk;
    const int slot = pos % c.capacity;
    l.k = (bh * c.capacity + slot) * D;
    l.v = bh * D * c.capacity + slot;
    l.si = static_cast<int>(bh);
    l.ok = true;
  } else {
    const int pi = pos / c.page_tokens;
    const int page = pi < c.max_pages ? c.block_table[static_cast<int64_t>(b) * c.max_pages + pi] : -1;
    l.ok = page >= 0 && page < c.num_pages;
    const int64_t ph = l.ok ? static_cast<int64_t>(page) * Hkv + hk : 0;
    const int row = pos - pi * c.page_tokens;
    l.k = (ph * c.page_tokens + row) * D;
    l.v = ph * D * c.page_tokens + row;
    l.si = static_cast<int>(ph);
  }
  return l;
}

__device__ __forceinline__ int cache_vstride(const CacheView& c) {
  return c.kind == MUSE_KV_RING ? c.capacity : c.page_tokens;
}

// ---------------------------------------------------------------------------
// Chunked prefill, a tile whose 64 positions are all visible cached history:
// the image is a format change of the cache's own rows.  Key rows widen to
// fp32 (E4M3 codes times their scale) and narrow to fp16; a value image
// chunk holds keys 0-3 and 8-11 (or 4-7 and 12-15) of a 16-position group,
// i.e. one half of each of two 8-position runs of the cache's head-dim-major
// rows, so it is assembled in registers from two cache reads.  The same
// arithmetic as the general path below; absent pages give zeros.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void kv_prep_history_tile(const KvPrepArgs& a, int b, int hk, int pos0, u32x4* tdst,
                                                     float* kss, int64_t tile_index) {
  using TL = TileLayout<D>;
  constexpr int BK = kKeyTile;
  constexpr int KC = D / 8;
  const int tid = threadIdx.x;
  const CacheView& cv = a.cache;
  // keys: KC consecutive lanes carry the KC chunks of one row (their sum of
  // squares is a reduction over the group)
  float mrow = 0.f;
  for (int j = tid; j < BK * KC; j += 256) {
    const int r = j / KC, c = j - r * KC;
    u32x4 out = {0, 0, 0, 0};
    float s2 = 0.f;
    const CacheLoc cl = cache_loc(cv, b, hk, a.Hkv, D, pos0 + r);
    if (cl.ok) {
      float f[8];
      const int64_t off = cl.k + c * 8;
      if (cv.fp8) {
        unpack_bf16x8(e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(cv.k) + off)), f);
        const float sc = cv.k_scale[cl.si];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= sc;
      } else {
        unpack_bf16x8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(cv.k) + off), f);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s2 += f[e] * f[e];
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = pack_f16x2(f[2 * i], f[2 * i + 1]);
    }
    mrow = fmaxf(mrow, group_sum<KC>(s2) * (1.0f / D));
    tdst[TL::k(r, c)] = out;
  }
  // the tile's largest key mean square (every row is visible history)
  mrow = wave_max(mrow);
  if ((tid & 63) == 0) kss[tid >> 6] = mrow;
  __syncthreads();
  if (tid == 0) a.tile_ms[tile_index] = fmaxf(fmaxf(kss[0], kss[1]), fmaxf(kss[2], kss[3]));
  // values: item (d, g16) writes image chunks 2 g16 and 2 g16 + 1 of head-dim row d
  const int vstride = cache_vstride(cv);
  for (int it = tid; it < D * (BK / 16); it += 256) {
    const int d = it / (BK / 16), g16 = it - d * (BK / 16);
    const CacheLoc cl = cache_loc(cv, b, hk, a.Hkv, D, pos0 + 16 * g16);
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};  // positions 0-7 and 8-15 of the group, bf16 pairs
    if (cl.ok) {
      const int64_t off = cl.v + static_cast<int64_t>(d) * vstride;
      if (cv.fp8) {
        const float sc = cv.v_scale[cl.si];
        const uint8_t* src = static_cast<const uint8_t*>(cv.v) + off;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float f[8];
          unpack_bf16x8(e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(src + 8 * h)), f);
          u32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = static_cast<uint32_t>(f32_to_bf16_bits(f[2 * i] * sc)) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(f[2 * i + 1] * sc)) << 16);
          if (h == 0) x = w;
          else y = w;
        }
      } else {
        const uint16_t* src = static_cast<const uint16_t*>(cv.v) + off;
        x = *reinterpret_cast<const u32x4*>(src);
        y = *reinterpret_cast<const u32x4*>(src + 8);
      }
    }
    tdst[TL::v(d, 2 * g16)] = u32x4{x[0], x[1], y[0], y[1]};
    tdst[TL::v(d, 2 * g16 + 1)] = u32x4{x[2], x[3], y[2], y[3]};
  }
}

// ---------------------------------------------------------------------------
// Prefill key/value preparation: one 64-key tile of one (sequence, KV head)
// per workgroup.  Writes the tile image the attention kernel copies straight
// into LDS: k_hat as fp16 key rows and V transposed to head-dim rows (bf16),
// both with one pad chunk per row (layout in TileLayout).
// CHUNK (chunked prefill): tile rows are positions kbase + slot; rows the
// chunk's queries can see below the chunk start are read from the cache as
// stored (E4M3 codes times their scale), rows from the start on are the
// chunk's own keys and values.
// ---------------------------------------------------------------------------
template <int D, bool CHUNK>
__global__ __launch_bounds__(256) void kv_prep_kernel(KvPrepArgs a) {
  constexpr int BK = kKeyTile;
  constexpr int RUN = D / 8;  // elements per thread in each half of the head
  __shared__ uint16_t vs[BK][D + 8];
  __shared__ float kss[BK];  // chunked prefill: cached key rows' sums of squares, then per-wave maxima
  // KV heads vary fastest over the grid: the workgroups of one tile's heads
  // run together and read each token's row of all heads in one pass
  const int tile = blockIdx.x / a.Hkv;
  const int hk = blockIdx.x - tile * a.Hkv;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int r = tid >> 2;          // key within the tile
  const int qq = tid & 3;          // quarter of each half of the head
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;

  // chunked prefill: the chunk start, the tile image's first position and
  // the first cached position any query of the chunk sees
  int st = 0, kb = 0, need_lo = 0;
  if constexpr (CHUNK) {
    st = a.start[b];
    if (!chunk_start_ok(st, a.max_start)) st = 0;
    kb = chunk_kbase(st, a.W);
    need_lo = a.W > 0 ? max(0, st - a.W + 1) : 0;
  }
  const int pos0 = kb + tile * BK;  // position of the tile's first row
  if constexpr (CHUNK) {
    // a tile of visible history only (uniform over the workgroup)
    if (pos0 >= need_lo && pos0 + BK <= st) {
      kv_prep_history_tile<D>(a, b, hk, pos0, a.tiles + (bh * a.n_tiles + tile) * TileLayout<D>::CHUNKS, kss,
                              bh * a.n_tiles + tile);
      return;
    }
  }
  const int tok = CHUNK ? pos0 + r - st : tile * BK + r;
  const bool hist = CHUNK && pos0 + r >= need_lo && pos0 + r < st;

  // All loads of the tile (raw keys, values and RoPE rows) are issued
  // before the first use so their latencies overlap.  Rows outside the
  // chunk repeat its first or last row: they are never visible to a query
  // (the attention kernel masks them before the exponential), and finite
  // values keep p = 0 from meeting a non-finite V.
  const int tl = min(max(tok, 0), a.T - 1);
  const uint16_t* kp = a.k + b * a.k_sb + static_cast<int64_t>(tl) * a.k_st + static_cast<int64_t>(hk) * D;
  const uint16_t* vp = a.v + b * a.v_sb + static_cast<int64_t>(tl) * a.v_st + static_cast<int64_t>(hk) * D;
  u32x4 kw[2][RUN / 8], vw[2][RUN / 8];
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      kw[hf][c] = *reinterpret_cast<const u32x4*>(kp + hf * (D / 2) + qq * RUN + c * 8);
      vw[hf][c] = *reinterpret_cast<const u32x4*>(vp + hf * (D / 2) + qq * RUN + c * 8);
    }
  float2 cs[RUN];
  const bool use_rope = a.rope != nullptr;
  if (use_rope) {
    const float2* rt = a.rope + ((a.rope_batched ? static_cast<int64_t>(b) * a.T : 0) + tl) * (D / 2) + qq * RUN;
#pragma unroll
    for (int e = 0; e < RUN; ++e) cs[e] = rt[e];
  }
  // cached key row of a history position, widened to bf16 bits
  u32x4 hw[2][RUN / 8];
  float hscale = 1.f;
  bool hok = false;
  if constexpr (CHUNK) {
    if (hist) {
      const CacheLoc cl = cache_loc(a.cache, b, hk, a.Hkv, D, pos0 + r);
      hok = cl.ok;
      if (hok) {
#pragma unroll
        for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int64_t off = cl.k + hf * (D / 2) + qq * RUN + c * 8;
            if (a.cache.fp8)
              hw[hf][c] = e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(a.cache.k) + off));
            else
              hw[hf][c] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.cache.k) + off);
          }
        if (a.cache.fp8) hscale = a.cache.k_scale[cl.si];
      }
    }
  }

  // ---- values: stage the tile for the transposed write ----
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      *reinterpret_cast<u32x2*>(&vs[r][hf * (D / 2) + qq * RUN + c * 8]) = u32x2{vw[hf][c][0], vw[hf][c][1]};
      *reinterpret_cast<u32x2*>(&vs[r][hf * (D / 2) + qq * RUN + c * 8 + 4]) = u32x2{vw[hf][c][2], vw[hf][c][3]};
    }

  // ---- keys: norm + RoPE, fp16 out ----
  float lo[RUN], hi[RUN];
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c) {
    unpack_16x8(kw[0][c], lo + c * 8, a.k_f16);
    unpack_16x8(kw[1][c], hi + c * 8, a.k_f16);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < RUN; ++e) ss += lo[e] * lo[e] + hi[e] * hi[e];
  ss = group_sum<4>(ss);
  const float rs = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    float x0 = lo[e] * rs, x1 = hi[e] * rs;
    if (use_rope) {
      const float y0 = x0 * cs[e].x - x1 * cs[e].y;
      const float y1 = x1 * cs[e].x + x0 * cs[e].y;
      x0 = y0;
      x1 = y1;
    }
    lo[e] = x0;
    hi[e] = x1;
  }
  if constexpr (CHUNK) {
    float hss = 0.f;
    if (hist) {
      // cached keys are taken as stored (absent pages read as zeros)
#pragma unroll
      for (int c = 0; c < RUN / 8; ++c) {
        float hl[8], hh[8];
        unpack_bf16x8(hw[0][c], hl);
        unpack_bf16x8(hw[1][c], hh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lo[c * 8 + e] = hok ? hl[e] * hscale : 0.f;
          hi[c * 8 + e] = hok ? hh[e] * hscale : 0.f;
          hss += lo[c * 8 + e] * lo[c * 8 + e] + hi[c * 8 + e] * hi[c * 8 + e];
        }
      }
    }
    // the tile's largest cached-key mean square: the row's four lanes, then
    // the wave, then (after the barrier below) the four waves
    const float wm = wave_max(group_sum<4>(hss) * (1.0f / D));
    if ((tid & 63) == 0) kss[tid >> 6] = wm;
  }
  using TL = TileLayout<D>;
  u32x4* tdst = a.tiles + (bh * a.n_tiles + tile) * TL::CHUNKS;
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c) {
    u32x4 w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = pack_f16x2(lo[c * 8 + 2 * i], lo[c * 8 + 2 * i + 1]);
      w1[i] = pack_f16x2(hi[c * 8 + 2 * i], hi[c * 8 + 2 * i + 1]);
    }
    const int c0 = (qq * RUN) / 8 + c;             // logical chunk, first half
    const int c1 = (D / 2 + qq * RUN) / 8 + c;     // logical chunk, second half
    tdst[TL::k(r, c0)] = w0;
    tdst[TL::k(r, c1)] = w1;
  }

  __syncthreads();
  if constexpr (CHUNK) {
    if (tid == 0) a.tile_ms[bh * a.n_tiles + tile] = fmaxf(fmaxf(kss[0], kss[1]), fmaxf(kss[2], kss[3]));
  }
  constexpr int CHUNKS = D * BK / 8;  // 16-byte chunks of the transposed tile
  if constexpr (CHUNK) {
    // cached values of history positions overwrite their staged rows; the
    // cache holds them head-dim-major, eight consecutive positions (one
    // page or ring run: pages and the ring hold multiples of 16) per read
    if (pos0 + BK > need_lo && pos0 < st) {
      const int vstride = cache_vstride(a.cache);
      for (int ci = tid; ci < CHUNKS; ci += 256) {
        const int d = ci / (BK / 8);
        const int g8 = ci % (BK / 8);
        const int p0 = pos0 + 8 * g8;
        if (p0 + 8 <= need_lo || p0 >= st) continue;
        const CacheLoc cl = cache_loc(a.cache, b, hk, a.Hkv, D, p0);
        uint16_t e[8];
        if (cl.ok) {
          const int64_t off = cl.v + static_cast<int64_t>(d) * vstride;
          if (a.cache.fp8) {
            const u32x4 w = e4m3x8_to_bf16x8(*reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(a.cache.v) + off));
            float f[8];
            unpack_bf16x8(w, f);
            const float sc = a.cache.v_scale[cl.si];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = f32_to_bf16_bits(f[i] * sc);
          } else {
            const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.cache.v) + off);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              e[2 * i] = static_cast<uint16_t>(w[i] & 0xffffu);
              e[2 * i + 1] = static_cast<uint16_t>(w[i] >> 16);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = 0;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (p0 + i >= need_lo && p0 + i < st) vs[8 * g8 + i][d] = e[i];
      }
      __syncthreads();
    }
  }
  // consecutive lanes write consecutive head-dim rows of one chunk: whole
  // lines of the chunk-major image
  for (int ci = tid; ci < CHUNKS; ci += 256) {
    const int d = ci % D;
    const int pc = ci / D;  // chunk: 16-key group g16 = pc/2, half hh = pc%2
    const int g16 = pc >> 1, hh = pc & 1;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = g16 * 16 + 4 * hh + (i & 3) + 8 * (i >> 2);
      e[i] = vs[key][d];
    }
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = static_cast<uint32_t>(e[2 * i]) | (static_cast<uint32_t>(e[2 * i + 1]) << 16);
    tdst[TL::v(d, pc)] = w;
  }
}

// ---------------------------------------------------------------------------
// Chunked prefill, cache write: the chunk's keys (norm + RoPE in fp32, then
// bf16 or the E4M3 code of key / scale) and values go to their positions.
// A ring keeps only the last W positions, so only the chunk's last min(T, W)
// rows are written (earlier ones would be overwritten within the call).
// One 64-row tile of one (sequence, KV head) per workgroup.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void chunk_append_kernel(ChunkAppendArgs a) {
  constexpr int BK = kKeyTile;
  constexpr int RUN = D / 8;
  __shared__ uint16_t vs[BK][D + 8];
  const int tile = blockIdx.x / a.Hkv;
  const int hk = blockIdx.x - tile * a.Hkv;
  const int b = blockIdx.y;
  const int st = a.start[b];
  if (!chunk_start_ok(st, a.max_start)) return;  // the whole workgroup
  const int tid = threadIdx.x;
  const int r = tid >> 2;
  const int qq = tid & 3;
  const int t = tile * BK + r;
  const int wlo = a.cache.kind == MUSE_KV_RING ? max(0, a.T - a.cache.capacity) : 0;
  const int tl = min(t, a.T - 1);
  const uint16_t* kp = a.k + b * a.k_sb + static_cast<int64_t>(tl) * a.k_st + static_cast<int64_t>(hk) * D;
  const uint16_t* vp = a.v + b * a.v_sb + static_cast<int64_t>(tl) * a.v_st + static_cast<int64_t>(hk) * D;
  u32x4 kw[2][RUN / 8], vw[2][RUN / 8];
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      kw[hf][c] = *reinterpret_cast<const u32x4*>(kp + hf * (D / 2) + qq * RUN + c * 8);
      vw[hf][c] = *reinterpret_cast<const u32x4*>(vp + hf * (D / 2) + qq * RUN + c * 8);
    }
  float2 cs[RUN];
  const bool use_rope = a.rope != nullptr;
  if (use_rope) {
    const float2* rt = a.rope + (static_cast<int64_t>(b) * a.T + tl) * (D / 2) + qq * RUN;
#pragma unroll
    for (int e = 0; e < RUN; ++e) cs[e] = rt[e];
  }
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      *reinterpret_cast<u32x2*>(&vs[r][hf * (D / 2) + qq * RUN + c * 8]) = u32x2{vw[hf][c][0], vw[hf][c][1]};
      *reinterpret_cast<u32x2*>(&vs[r][hf * (D / 2) + qq * RUN + c * 8 + 4]) = u32x2{vw[hf][c][2], vw[hf][c][3]};
    }

  float lo[RUN], hi[RUN];
#pragma unroll
  for (int c = 0; c < RUN / 8; ++c) {
    unpack_bf16x8(kw[0][c], lo + c * 8);
    unpack_bf16x8(kw[1][c], hi + c * 8);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < RUN; ++e) ss += lo[e] * lo[e] + hi[e] * hi[e];
  ss = group_sum<4>(ss);
  const float rs = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    float x0 = lo[e] * rs, x1 = hi[e] * rs;
    if (use_rope) {
      const float y0 = x0 * cs[e].x - x1 * cs[e].y;
      const float y1 = x1 * cs[e].x + x0 * cs[e].y;
      x0 = y0;
      x1 = y1;
    }
    lo[e] = x0;
    hi[e] = x1;
  }
  if (t < a.T && t >= wlo) {
    const CacheLoc cl = cache_loc(a.cache, b, hk, a.Hkv, D, st + t);
    if (cl.ok) {
      if (a.cache.fp8) {
        const float ks = a.cache.k_scale[cl.si];
        uint8_t* kc = static_cast<uint8_t*>(a.cache.k) + cl.k;
#pragma unroll
        for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const float* x = (hf ? hi : lo) + c * 8;
            u32x2 w = {0u, 0u};
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i >> 2] |= static_cast<uint32_t>(e4m3_encode(x[i] / ks)) << (8 * (i & 3));
            *reinterpret_cast<u32x2*>(kc + hf * (D / 2) + qq * RUN + c * 8) = w;
          }
      } else {
        uint16_t* kc = static_cast<uint16_t*>(a.cache.k) + cl.k;
#pragma unroll
        for (int c = 0; c < RUN / 8; ++c)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const float* x = (hf ? hi : lo) + c * 8;
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
            *reinterpret_cast<u32x4*>(kc + hf * (D / 2) + qq * RUN + c * 8) = w;
          }
      }
    }
  }
  __syncthreads();
  // values, head-dim-major in the cache: consecutive lanes take consecutive
  // positions of one dimension
  const int vstride = cache_vstride(a.cache);
  for (int ci = tid; ci < BK * D; ci += 256) {
    const int d = ci / BK;
    const int rr = ci - d * BK;
    const int tt = tile * BK + rr;
    if (tt >= a.T || tt < wlo) continue;
    const CacheLoc cl = cache_loc(a.cache, b, hk, a.Hkv, D, st + tt);
    if (!cl.ok) continue;
    const int64_t off = cl.v + static_cast<int64_t>(d) * vstride;
    if (a.cache.fp8)
      static_cast<uint8_t*>(a.cache.v)[off] = e4m3_encode(bf16_bits_to_f32(vs[rr][d]) / a.cache.v_scale[cl.si]);
    else
      static_cast<uint16_t*>(a.cache.v)[off] = vs[rr][d];
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
hipError_t launch_rope_qknorm(int d, int out_dtype, const RopeQkArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const int lpr = d / 2;
  const int64_t threads = a.n_rows * lpr;
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
#define MUSE_RQ(DD, OO) hipLaunchKernelGGL((rope_qknorm_kernel<DD, OO>), dim3(blocks), dim3(256), 0, st, a)
  if (d == 64) {
    if (out_dtype == MUSE_DTYPE_F32) MUSE_RQ(64, MUSE_DTYPE_F32);
    else if (out_dtype == MUSE_DTYPE_F16) MUSE_RQ(64, MUSE_DTYPE_F16);
    else MUSE_RQ(64, MUSE_DTYPE_BF16);
  } else {
    if (out_dtype == MUSE_DTYPE_F32) MUSE_RQ(128, MUSE_DTYPE_F32);
    else if (out_dtype == MUSE_DTYPE_F16) MUSE_RQ(128, MUSE_DTYPE_F16);
    else MUSE_RQ(128, MUSE_DTYPE_BF16);
  }
#undef MUSE_RQ
  return hipGetLastError();
}

hipError_t launch_rope_table(int d, const RopeTableArgs& a, hipStream_t st) {
  const int64_t n = a.n_rows * (d / 2);
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (d == 64) hipLaunchKernelGGL((rope_table_kernel<64>), dim3(blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((rope_table_kernel<128>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_prep(int d, int B, const KvPrepArgs& a, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(a.n_tiles) * static_cast<unsigned>(a.Hkv), B);
  if (a.start) {
    if (d == 64) hipLaunchKernelGGL((kv_prep_kernel<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((kv_prep_kernel<128, true>), grid, dim3(256), 0, st, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((kv_prep_kernel<64, false>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((kv_prep_kernel<128, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_append(int d, int B, const ChunkAppendArgs& a, hipStream_t st) {
  const unsigned tiles = static_cast<unsigned>((a.T + kKeyTile - 1) / kKeyTile);
  dim3 grid(tiles * static_cast<unsigned>(a.Hkv), B);
  if (d == 64) hipLaunchKernelGGL((chunk_append_kernel<64>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((chunk_append_kernel<128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace muse
