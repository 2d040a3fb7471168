// Decode: one new token per sequence against a ring (local layer) or paged
// (global layer) KV cache.
//
// What it computes (Muse Spark Open deep dive): the new token's q and k get
// the weightless QK-norm, the query multiplier and (local layers) RoPE at
// position p = kv_len - 1 (section 3.2 steps 2-4, section 3.4); the cache is
// updated after those steps (section 3.2 notes), a local layer keeps the W
// most recent entries (section 3.4 mask and cache notes, section 7.2), and
// the query attends to every visible entry (GQA, section 3.1), followed by
// Spark's per-head output norm and the sigmoid gate (section 3.3).
//
// Three kernels on the caller's stream:
//   1. append: prologue of the new token; q_hat (fp32, in log2 units) and
//      k_hat (fp32) to the workspace, k_hat and v (bf16) into the cache slot;
//   2. split: a grid of (sequence, KV head, chunk of cached entries) items;
//      each streams its chunk's K and V with 16-byte loads straight into MFMA
//      operands and keeps a running maximum (the cache is caller data, so no
//      bound on its logits is assumed); partial (max, sum, O) per item;
//   3. combine: merges the partials with the new token's own term (computed
//      in fp32 from the workspace copies), then output norm and gate.
// Both contractions run on v_mfma_f32_16x16x32_bf16.  To keep fp32 accuracy
// with bf16 operands, q_hat and p are split into hi + lo bf16 parts whose two
// products accumulate into the same fp32 registers (the MFMA work this
// doubles is far below the HBM roofline that bounds decode).
#include <type_traits>

#include "kernels.h"

namespace muse {

__device__ __forceinline__ bool decode_len_ok(int L, int max_len) { return L >= 1 && L <= max_len; }

// ---------------------------------------------------------------------------
// 1. append
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_append_kernel(DecodeArgs a, int hq_total) {
  constexpr int LPR = D / 2;
  const int b = blockIdx.y;
  const int L = a.kv_len[b];
  const bool len_ok = decode_len_ok(L, a.max_kv_len);
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = gt / LPR;              // 0 .. Hq-1: queries; Hq .. Hq+Hkv-1: keys
  const int j = gt % LPR;
  const int rows = hq_total + a.Hkv;
  const bool valid = row < rows;
  const bool is_q = row < hq_total;
  const int h = is_q ? row : row - hq_total;
  float x0 = 0.f, x1 = 0.f;
  if (valid) {
    const uint16_t* p = is_q ? a.q_new + b * a.q_sb + static_cast<int64_t>(h) * D
                             : a.k_new + b * a.kv_sb + static_cast<int64_t>(h) * D;
    x0 = bits16_to_f32(p[j], a.in_f16);
    x1 = bits16_to_f32(p[j + D / 2], a.in_f16);
  }
  const float ss = group_sum<LPR>(x0 * x0 + x1 * x1);
  const float r = (is_q ? a.qscale : 1.0f) / sqrtf(ss * (1.0f / D) + a.qk_eps);
  x0 *= r;
  x1 *= r;
  const int pos = len_ok ? L - 1 : 0;
  if (a.use_rope) {
    float s, c;
    rope_sincos(pos, j, D, a.log2_theta, &s, &c);
    const float y0 = x0 * c - x1 * s;
    const float y1 = x1 * c + x0 * s;
    x0 = y0;
    x1 = y1;
  }
  if (!valid) return;
  if (is_q) {
    float* qo = a.qhat + (static_cast<int64_t>(b) * hq_total + h) * D;
    qo[j] = x0;
    qo[j + D / 2] = x1;
    return;
  }
  float* ko = a.khat + (static_cast<int64_t>(b) * a.Hkv + h) * D;
  ko[j] = x0;
  ko[j + D / 2] = x1;
  if (!len_ok) return;
  // cache write: k_hat row (token-major) and v column (head-dim-major)
  const uint16_t* vp = a.v_new + b * a.kv_sb + static_cast<int64_t>(h) * D;
  int64_t kbase, vbase, vstride;
  if (a.kind == MUSE_KV_RING) {
    const int slot = pos % a.capacity;
    kbase = ((static_cast<int64_t>(b) * a.Hkv + h) * a.capacity + slot) * D;
    vbase = (static_cast<int64_t>(b) * a.Hkv + h) * D * a.capacity + slot;
    vstride = a.capacity;
  } else {
    const int pi = pos / a.page_tokens;
    const int rr = pos % a.page_tokens;
    const int64_t page = a.block_table[static_cast<int64_t>(b) * a.max_pages + pi];
    if (page < 0 || page >= a.num_pages) return;
    kbase = ((page * a.Hkv + h) * a.page_tokens + rr) * D;
    vbase = (page * a.Hkv + h) * D * a.page_tokens + rr;
    vstride = a.page_tokens;
  }
  if (a.fp8) {
    // E4M3 codes of x / scale, the division in IEEE fp32 (per-(page, head)
    // or per-(sequence, head) scales)
    const int64_t si = a.kind == MUSE_KV_RING ? static_cast<int64_t>(b) * a.Hkv + h
                                              : (kbase / D / a.page_tokens);  // page * Hkv + h
    const float ks = a.k_scale[si], vs = a.v_scale[si];
    uint8_t* kc8 = reinterpret_cast<uint8_t*>(a.kc);
    uint8_t* vc8 = reinterpret_cast<uint8_t*>(a.vc);
    kc8[kbase + j] = e4m3_encode(x0 / ks);
    kc8[kbase + j + D / 2] = e4m3_encode(x1 / ks);
    vc8[vbase + static_cast<int64_t>(j) * vstride] = e4m3_encode(bf16_bits_to_f32(vp[j]) / vs);
    vc8[vbase + static_cast<int64_t>(j + D / 2) * vstride] = e4m3_encode(bf16_bits_to_f32(vp[j + D / 2]) / vs);
    return;
  }
  a.kc[kbase + j] = f32_to_bf16_bits(x0);
  a.kc[kbase + j + D / 2] = f32_to_bf16_bits(x1);
  a.vc[vbase + static_cast<int64_t>(j) * vstride] = vp[j];
  a.vc[vbase + static_cast<int64_t>(j + D / 2) * vstride] = vp[j + D / 2];
}

// Visible cached entries of sequence b, as an index range with a validity test.
struct HistRange {
  int base;   // first index of chunk 0
  int end;    // indices < end may be valid
  int lo;     // paged: first visible position
  int skip;   // ring: slot holding the new token (excluded), or -1
};

__device__ __forceinline__ HistRange hist_range(const DecodeArgs& a, int L) {
  HistRange r;
  if (a.kind == MUSE_KV_RING) {
    r.base = 0;
    r.lo = 0;
    if (L >= a.capacity) {
      r.end = a.capacity;
      r.skip = (L - 1) % a.capacity;
    } else {
      r.end = L - 1;
      r.skip = -1;
    }
  } else {
    r.lo = a.W > 0 ? max(0, L - a.W) : 0;
    r.base = (r.lo / a.chunk_tokens) * a.chunk_tokens;
    r.end = L - 1;
    r.skip = -1;
  }
  return r;
}

__device__ __forceinline__ int hist_chunks(const HistRange& r, int chunk_tokens) {
  return r.end > r.base ? (r.end - r.base + chunk_tokens - 1) / chunk_tokens : 0;
}

__device__ __forceinline__ bool hist_valid(const HistRange& r, int idx) {
  return idx < r.end && idx >= r.lo && idx != r.skip;
}

// ---------------------------------------------------------------------------
// 2. split
// ---------------------------------------------------------------------------
// 8-entry blocks of the largest paged chunk (each lies inside one page: pages
// hold a multiple of 16 positions and chunks start at multiples of 8).
constexpr int kChunkBlocks = kPagedChunkMax / 8;
// Register buffers of 32-entry sub-chunks per wave (PD - 1 in flight).  bf16
// keeps two in flight: a cold 2048-entry ring then overlaps more of its load
// latency (measured 5 % faster; the same on pages), while a fourth buffer
// measured 11 % slower on the ring.  The E4M3 loop is bound by instruction
// issue: three or four buffers measured 1.5 % and 4 % slower there.
constexpr int kDecodeDepth = 3;
constexpr int kDecodeDepthFp8 = 2;
// The running maximum (log2 units) is raised only when a logit exceeds it by
// more than this, so unnormalized weights stay below 2^kRescaleSlack and most
// sub-chunks skip the rescale of the accumulators.
constexpr float kRescaleSlack = 16.f;

template <int D, int G, bool FP8>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int NW = 4;
  constexpr int DS = D / 32;  // dim steps of QK^T
  constexpr int DB = D / 16;  // dim blocks of O^T
  constexpr float NEG = -1.0e30f;
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ float sm_o[NW][16][D + 1];
  // paged: element offsets of each 8-entry block's first K row and first V
  // column (-1: page absent) and its scale index page * Hkv + hk
  __shared__ int64_t sm_koff[kChunkBlocks];
  __shared__ int64_t sm_voff[kChunkBlocks];
  __shared__ int sm_sidx[kChunkBlocks];

  const int item = blockIdx.x;
  const int c = item % a.max_chunks;
  const int bh = item / a.max_chunks;
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const int L = a.kv_len[b];
  if (!decode_len_ok(L, a.max_kv_len)) return;
  const HistRange hr = hist_range(a, L);
  if (c >= hist_chunks(hr, a.chunk_tokens)) return;
  const int c0 = hr.base + c * a.chunk_tokens;
  const int c1 = min(c0 + a.chunk_tokens, hr.end);

  const int tid = threadIdx.x;
  // wave index as a wave-uniform (scalar) value: the sub-chunk loop and its
  // full / partial test then branch on scalars instead of lane masks
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;  // query head within the group (columns >= G are padding)
  const int g4 = lane >> 4;   // 0..3

  // q_hat hi/lo operands (B of S^T = K Q^T): head col, dims 8*g4 + 32*ds + [0, 8)
  bf16x8 qhi[DS], qlo[DS];
  {
    const float* qp = a.qhat + (static_cast<int64_t>(b) * (a.Hkv * G) + hk * G + (col < G ? col : 0)) * D + 8 * g4;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (col < G) {
        x0 = *reinterpret_cast<const f32x4*>(qp + 32 * ds);
        x1 = *reinterpret_cast<const f32x4*>(qp + 32 * ds + 4);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? x0[e] : x1[e - 4];
        const bf16_t hi = static_cast<bf16_t>(x);
        qhi[ds][e] = hi;
        qlo[ds][e] = static_cast<bf16_t>(x - static_cast<float>(hi));
      }
    }
  }

  // Paged cache: the page lookup of every block is done once per workgroup
  // (one block per thread), so a prefetch address is one LDS read away
  // instead of a division and a dependent global load (whose wait would also
  // drain the loads already in flight).
  const bool paged = a.kind != MUSE_KV_RING;
  const int pt = a.page_tokens;
  if (paged) {
    for (int i = tid; i < a.chunk_tokens / 8; i += NW * kWave) {
      const int idx = c0 + 8 * i;
      int64_t ko = -1, vo = -1;
      int si = -1;
      if (idx < c1) {
        const int pi = idx / pt;
        const int r = idx - pi * pt;
        const int page = pi < a.max_pages ? a.block_table[static_cast<int64_t>(b) * a.max_pages + pi] : -1;
        if (page >= 0 && page < a.num_pages) {
          si = page * a.Hkv + hk;
          ko = (static_cast<int64_t>(si) * pt + r) * D;
          vo = static_cast<int64_t>(si) * D * pt + r;
        }
      }
      sm_koff[i] = ko;
      sm_voff[i] = vo;
      sm_sidx[i] = si;
    }
    __syncthreads();
  }

  const uint16_t* kc = a.kc;
  const uint16_t* vc = a.vc;
  const int vstride = paged ? pt : a.capacity;

  float m = NEG, lsum = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Sub-chunks of 32 entries stream through PD register buffers: while one is
  // processed, the next PD - 1 are in flight.  The loop is unrolled by PD so
  // every buffer index is a compile-time constant (no register copies, whose
  // waits would drain the loads in flight).  Row r = 4g + i of key tile kt
  // holds entry 8g + 4kt + i, so the eight entries a lane needs for P V are
  // contiguous in the head-dim-major V rows (one 16-byte load per fragment).
  // A lane's K rows lie in 8-entry block col / 4 of the sub-chunk, its logits,
  // weights and V entries in block g4.
  constexpr int PD = FP8 ? kDecodeDepthFp8 : kDecodeDepth;
  // one fragment: 8 entries of 16 bits (bf16) or 8 bits (E4M3 codes)
  using Frag = typename std::conditional<FP8, u32x2, u32x4>::type;
  struct Buf {
    Frag k[2][DS];
    Frag v[DB];
    bool kok, vok;
    float ks, vs;  // E4M3: scales of the page holding this lane's entries
  };
  Buf bufs[PD];
  const uint8_t* kc8 = reinterpret_cast<const uint8_t*>(a.kc);
  const uint8_t* vc8 = reinterpret_cast<const uint8_t*>(a.vc);
  // Loads are issued unconditionally (an absent block reads the start of the
  // cache instead) and zeroed at use: predicated loads would leave the
  // number of loads in flight unknown and force full waits.
  auto load = [&](Buf& B, int s0) {
    int64_t ka, va;
    if (paged) {
      const int blk = (s0 - c0) >> 3;
      const int64_t ko = sm_koff[blk + (col >> 2)];
      const int64_t vo = sm_voff[blk + g4];
      B.kok = ko >= 0;
      B.vok = vo >= 0;
      ka = B.kok ? ko + (col & 3) * D : 0;
      va = B.vok ? vo : 0;
    } else {
      const int ik = s0 + 8 * (col >> 2);
      const int iv = s0 + 8 * g4;
      B.kok = ik < hr.end;
      B.vok = iv < hr.end;
      ka = B.kok ? (static_cast<int64_t>(bh) * a.capacity + ik + (col & 3)) * D : 0;
      va = B.vok ? static_cast<int64_t>(bh) * D * a.capacity + iv : 0;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        if constexpr (FP8)
          B.k[kt][ds] = *reinterpret_cast<const u32x2*>(kc8 + ka + 4 * kt * D + 32 * ds + 8 * g4);
        else
          B.k[kt][ds] = *reinterpret_cast<const u32x4*>(kc + ka + 4 * kt * D + 32 * ds + 8 * g4);
      }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (FP8)
        B.v[db] = *reinterpret_cast<const u32x2*>(vc8 + va + static_cast<int64_t>(16 * db + col) * vstride);
      else
        B.v[db] = *reinterpret_cast<const u32x4*>(vc + va + static_cast<int64_t>(16 * db + col) * vstride);
    }
    if constexpr (FP8) {
      // issued for both cache kinds so every path has the same loads in flight
      const int si = paged ? max(sm_sidx[((s0 - c0) >> 3) + g4], 0) : bh;
      B.ks = a.k_scale[si];
      B.vs = a.v_scale[si];
    }
  };

  auto process = [&](Buf& B, int s0) {
    // A sub-chunk whose 32 entries are all visible, written and present (the
    // common case) skips every per-entry mask; the test is wave-uniform.
    const bool full = s0 >= hr.lo && s0 + 32 <= hr.end && (hr.skip < s0 || hr.skip >= s0 + 32) &&
                      __builtin_amdgcn_ballot_w64(!(B.kok && B.vok)) == 0;
    u32x4 kcur[2][DS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        if constexpr (FP8)
          kcur[kt][ds] = e4m3x8_to_bf16x8(B.k[kt][ds]);
        else
          kcur[kt][ds] = B.k[kt][ds];
      }
    u32x4 vcur[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (FP8)
        vcur[db] = e4m3x8_to_bf16x8(B.v[db]);
      else
        vcur[db] = B.v[db];
    }
    if (!full) {
      // absent blocks read as zeros; V entries at or past the end may never
      // have been written and are zeroed too, so p = 0 never meets a
      // non-finite value
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          if (!B.kok) kcur[kt][ds] = u32x4{0, 0, 0, 0};
      const int nv = B.vok ? hr.end - (s0 + 8 * g4) : 0;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
          vcur[db][wd] = 2 * wd >= nv ? 0u : (2 * wd + 1 >= nv ? (vcur[db][wd] & 0xffffu) : vcur[db][wd]);
    }
    const float kscale = FP8 ? B.ks : 1.f;
    const float vscale = FP8 ? B.vs : 1.f;

    // S^T tiles: entries s0 + 8*g4 + 4*kt + i, head col
    float s[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, kcur[kt][ds]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qhi[ds], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[ds], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kt][i] = FP8 ? acc[i] * kscale : acc[i];
    }
    if (!full) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!hist_valid(hr, s0 + 8 * g4 + 4 * kt + i)) s[kt][i] = NEG;
    }
    float tmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    if (__builtin_amdgcn_ballot_w64(tmax > m + kRescaleSlack) != 0) {
      // the lanes of one column (head) share its maximum
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float mnew = fmaxf(m, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    float p[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[kt][i] = __builtin_amdgcn_exp2f(s[kt][i] - m);
    if (!full) {
      // masked entries of a column that has seen no visible entry yet
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(s[kt][i] > NEG)) p[kt][i] = 0.f;
    }
    bf16x8 phi, plo;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        psum += p[kt][i];
        const float pv = FP8 ? p[kt][i] * vscale : p[kt][i];  // the value scale of this lane's page
        const bf16_t hi = static_cast<bf16_t>(pv);
        phi[4 * kt + i] = hi;
        plo[4 * kt + i] = static_cast<bf16_t>(pv - static_cast<float>(hi));
      }
    lsum += psum;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 vf = __builtin_bit_cast(bf16x8, vcur[db]);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi, o[db], 0, 0, 0);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo, o[db], 0, 0, 0);
    }
  };

  // this wave's sub-chunks: w, w + NW, w + 2 NW, ...  Every prefetch is
  // issued, past the end as a repeat of the last sub-chunk, so the number
  // of loads in flight is the same on every path through the loop.
  const int nsub = (c1 - c0 + 31) / 32;
  const int nmine = nsub > w ? (nsub - w + NW - 1) / NW : 0;
  auto sub_s0 = [&](int j) { return c0 + 32 * (w + min(j, nmine - 1) * NW); };
  if (nmine > 0) {
#pragma unroll
    for (int j = 0; j < PD - 1; ++j) load(bufs[j], sub_s0(j));
    int j0 = 0;
    for (; j0 + PD <= nmine; j0 += PD) {
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        load(bufs[(u + PD - 1) % PD], sub_s0(j0 + u + PD - 1));
        process(bufs[u], sub_s0(j0 + u));
      }
    }
    // fewer than PD sub-chunks left, in bufs[0 .. PD - 2]
#pragma unroll
    for (int u = 0; u < PD - 1; ++u)
      if (j0 + u < nmine) process(bufs[u], sub_s0(j0 + u));
  }
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);

  // merge the waves' partials
  if (g4 == 0) {
    sm_m[w][col] = m;
    sm_l[w][col] = lsum;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][col][16 * db + 4 * g4 + i] = o[db][i];
  __syncthreads();
  float* part = a.part + (static_cast<int64_t>(bh) * a.max_chunks + c) * (G * (D + 2));
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, d = e % D;
    float mm = NEG;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, sm_m[ww][h]);
    float acc = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = sm_m[ww][h] > NEG ? __builtin_amdgcn_exp2f(sm_m[ww][h] - mm) : 0.f;
      acc += f * sm_o[ww][h][d];
      ls += f * sm_l[ww][h];
    }
    part[h * (D + 2) + d] = acc;
    if (d == 0) {
      part[h * (D + 2) + D] = mm;
      part[h * (D + 2) + D + 1] = ls;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. combine + epilogue: one workgroup per (sequence, KV head); wave w takes
// heads w, w + 4, ...; lane = dim (two dims per lane when D = 128).
// ---------------------------------------------------------------------------
// Combine: one workgroup per (sequence, KV head) merges the chunk partials
// of its G query heads and adds the new token's own term.  The chunks are
// spread over NWC waves (chunk c to wave c mod NWC) so their loads overlap:
// each wave first takes the maximum over its chunks of every head, then,
// after the workgroup's maximum is known, sums its chunks' rescaled partials;
// the waves' sums meet in LDS, and wave w finishes heads w, w + NWC, ...
// (1/sum, output norm, gate).
template <int D, int G>
struct CombineShape {
  static constexpr int NWC = G * D > 1024 ? 8 : 16;  // waves (LDS: NWC * G * D floats)
};

template <int D, int G>
__global__ __launch_bounds__((CombineShape<D, G>::NWC * 64)) void decode_combine_kernel(DecodeArgs a) {
  constexpr int NWC = CombineShape<D, G>::NWC;
  constexpr int PER = D / 64;
  constexpr int ROW = G * (D + 2);  // floats of one chunk's partial: per head O[D], m, l
  constexpr int CPI = 64 / G;       // chunks one wave reads per step of the maximum pass
  constexpr float NEG = -1.0e30f;
  static_assert(64 % G == 0, "the heads tile a wave");
  __shared__ float s_new[G];
  __shared__ float s_max[NWC][G];
  __shared__ float s_l[NWC][G];
  __shared__ float s_acc[NWC][G][D];
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int L = a.kv_len[b];
  const bool len_ok = decode_len_ok(L, a.max_kv_len);
  const int nch = len_ok ? hist_chunks(hist_range(a, L), a.chunk_tokens) : 0;
  const float* part = a.part + static_cast<int64_t>(bh) * a.max_chunks * ROW;

  // the new token's own logit (log2 units) of heads w, w + NWC, ...
  for (int g = w; g < G; g += NWC) {
    const float* qp = a.qhat + (static_cast<int64_t>(b) * a.Hkv * G + hk * G + g) * D;
    const float* kn = a.khat + static_cast<int64_t>(bh) * D;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) dot += qp[lane + 64 * e] * kn[lane + 64 * e];
    dot = wave_sum(dot);
    if (lane == 0) s_new[g] = dot;
  }
  // maximum over this wave's chunks: lane -> (head lane mod G, chunk lane / G)
  {
    const int g = lane % G;
    float m = NEG;
    for (int c = w * CPI + lane / G; c < nch; c += NWC * CPI)
      m = fmaxf(m, part[static_cast<int64_t>(c) * ROW + g * (D + 2) + D]);
#pragma unroll
    for (int off = G; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane < G) s_max[w][lane] = m;
  }
  __syncthreads();
  float mm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = s_new[g];
#pragma unroll
    for (int i = 0; i < NWC; ++i) x = fmaxf(x, s_max[i][g]);
    mm[g] = x;
  }
  // this wave's chunks, rescaled to the workgroup's maximum
  float acc[G][PER], ls[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    ls[g] = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[g][e] = 0.f;
  }
#pragma unroll 2
  for (int c = w; c < nch; c += NWC) {
    const float* pc = part + static_cast<int64_t>(c) * ROW;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mc = pc[g * (D + 2) + D];
      const float f = mc > NEG ? __builtin_amdgcn_exp2f(mc - mm[g]) : 0.f;
      ls[g] += f * pc[g * (D + 2) + D + 1];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[g][e] += f * pc[g * (D + 2) + lane + 64 * e];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < PER; ++e) s_acc[w][g][lane + 64 * e] = acc[g][e];
    if (lane == 0) s_l[w][g] = ls[g];
  }
  __syncthreads();
  // heads w, w + NWC, ...: the new token's term, the waves' sums, then the epilogue
  const uint16_t* vn = a.v_new + b * a.kv_sb + static_cast<int64_t>(hk) * D;
  for (int g = w; g < G; g += NWC) {
    const int hq = hk * G + g;
    const float fnew = __builtin_amdgcn_exp2f(s_new[g] - mm[g]);
    float l = fnew;
#pragma unroll
    for (int i = 0; i < NWC; ++i) l += s_l[i][g];
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      o[e] = fnew * bf16_bits_to_f32(vn[lane + 64 * e]);
#pragma unroll
      for (int i = 0; i < NWC; ++i) o[e] += s_acc[i][g][lane + 64 * e];
    }
    const float inv = 1.0f / l;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      o[e] *= inv;
      ss += o[e] * o[e];
    }
    float rsn = 1.0f;
    if (a.out_norm) rsn = 1.0f / sqrtf(wave_sum(ss) * (1.0f / D) + a.out_eps);
    const uint16_t* gp = a.gate + b * a.g_sb + static_cast<int64_t>(hq) * D;
    uint16_t* op = a.out + (static_cast<int64_t>(b) * a.Hkv * G + hq) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float gv = bits16_to_f32(gp[lane + 64 * e], a.in_f16);
      const float y = len_ok ? o[e] * rsn / (1.0f + __expf(-gv)) : 0.f;
      op[lane + 64 * e] = f32_to_bf16_bits(y);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {
template <int D, int G>
hipError_t launch_dg(const DecodeArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int hq = a.Hkv * G;
  const int rows = hq + a.Hkv;
  const int threads = rows * (D / 2);
  dim3 g1((threads + 255) / 256, a.B);
  hipLaunchKernelGGL((decode_append_kernel<D>), g1, dim3(256), 0, st, a, hq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned items = static_cast<unsigned>(a.B) * a.Hkv * a.max_chunks;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  if (a.fp8)
    hipLaunchKernelGGL((decode_split_kernel<D, G, true>), dim3(items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, G, false>), dim3(items), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, G>), dim3(a.B * a.Hkv), dim3(CombineShape<D, G>::NWC * 64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int g, const DecodeArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  switch (g) {
    case 1: return launch_dg<D, 1>(a, st, e0, e1);
    case 2: return launch_dg<D, 2>(a, st, e0, e1);
    case 4: return launch_dg<D, 4>(a, st, e0, e1);
    case 8: return launch_dg<D, 8>(a, st, e0, e1);
    case 16: return launch_dg<D, 16>(a, st, e0, e1);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_decode(int d, int g, const DecodeArgs& a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  return d == 64 ? launch_d<64>(g, a, st, e0, e1) : launch_d<128>(g, a, st, e0, e1);
}

}  // namespace muse
