// The block attention of a block-diffusion drafter (Muse Spark Open deep
// dive, section 8.2, the drafter's fourth step: the block's tokens attend to
// the cached context and to each other with no causal mask) as a decode of
// a few tokens at once, for blocks of at most 64 tokens whose T * G
// (token, head) query columns fit 128 per KV head.  Two kernels:
//   1. split: per (sequence, KV head, group of 64 columns) and chunk of the
//      cached context, one workgroup of four waves, 16 columns each.  It
//      forms the q_hat of its columns in registers (the weightless norm,
//      s * log2(e) / sqrt(D), RoPE at the token's position; section 3.2
//      steps 2-4, section 3.4), then streams its chunk through LDS in
//      64-entry sub-chunks: whole-line loads of the cache as stored (bf16,
//      or E4M3 codes widened to bf16 on the way), written to a swizzled
//      image that the four waves read their MFMA fragments from.  Position j
//      is visible to the token at P iff |P - j| < W (section 3.4 and the
//      drafter's two-sided window), so the first visible position depends
//      on the column.  The last workgroup of a sequence also takes the
//      block's own keys, normalized and rotated in fp32 and split into bf16
//      hi + lo, as one more sub-chunk.  Each workgroup writes a partial
//      (running max, sum, O) per column.
//   2. combine: merges the partials, then 1/sum, Spark's per-head output
//      norm and the sigmoid gate (section 3.3), bf16.
// Products are MFMA 16x16x32 bf16 with q_hat and p split into bf16 hi + lo
// parts (near-fp32 products).  The K rows of each 16-entry logit tile are
// read in a permuted order so that a lane's eight weights are eight
// consecutive entries, one 16-byte piece of the head-dim-major V image.  The
// softmax keeps a running maximum (raised lazily, by more than 16 log2
// units), so cached keys of any RMS are exact.
#include <type_traits>

#include "draft.h"

namespace muse {

namespace {
constexpr float kNeg = -1.0e30f;
constexpr float kSlack = 16.f;
constexpr int kSub = 64;          // entries per sub-chunk
constexpr int kWavesDraft = 4;    // split: 16 columns per wave; combine: heads per workgroup
constexpr int kBlkMax = kDraftChunkMax / 8;

// Image row of sub-chunk entry e = 32h + 8q + 4kt + i (q, i < 4): 32h + 16kt
// + 4q + i.  A logit tile (h, kt) reads its 16 K rows in the order 8q + 4kt
// + i, so that a lane's eight weights are eight consecutive entries; stored
// this way those rows are 16 consecutive image rows, which a row stride of
// KC + 1 chunks (KC: 16-byte chunks per row) spreads over 16 distinct bank
// groups, and every fragment address is a per-lane base plus a constant.
__device__ __forceinline__ int kperm(int e) {
  return (e & 32) | (((e >> 2) & 1) << 4) | (((e >> 3) & 3) << 2) | (e & 3);
}
constexpr int kVS = 9;   // V dim stride in chunks (eight chunks of eight entries, plus one)

// Head dim staged by V piece row r (r = piece / pieces per dim): the 16
// lanes of one LDS write take dims d and d + 8 (bf16: 8 pieces per dim) or
// d, d + 1, d + 8, d + 9 (E4M3: 4 pieces per dim, two chunks each), whose
// chunks fall in 16 distinct bank groups at the 9-chunk dim stride.
template <bool FP8>
__device__ __forceinline__ int vdim(int r) {
  if constexpr (FP8) {
    const int g = r >> 2, k = r & 3;
    return (g >> 2) * 16 + (g & 3) * 2 + (k & 1) + (k >> 1) * 8;
  } else {
    const int g = r >> 1;
    return (g >> 3) * 16 + (r & 1) * 8 + (g & 7);
  }
}

// Sixteen E4M3 codes (one 16-byte piece) to two chunks of eight bf16.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4 w, u32x4& lo, u32x4& hi) {
  lo = e4m3x8_to_bf16x8(u32x2{w[0], w[1]});
  hi = e4m3x8_to_bf16x8(u32x2{w[2], w[3]});
}
}  // namespace

// ---------------------------------------------------------------------------
// 1. split.  Block index = wgi * (B * Hkv * n_cgroups) + bh * n_cgroups + cg:
// workgroup wgi streams context positions [base + wgi * chunk, + chunk).  Lane (col,
// g4) of wave w: column cg * 64 + 16 w + col (col = lane & 15), g4 = lane >> 4.
// Image of a sub-chunk (16-byte chunks): K [64 rows][KC + 1] (chunk c of
// entry e at kperm(e) * (KC + 1) + c), then V [D dims][9] (entries 8c ..
// 8c + 7 of dim d at d * 9 + c).
// ---------------------------------------------------------------------------
template <int D, bool FP8>
__global__ __launch_bounds__(256) void draft_split_kernel(DraftArgs a) {
  constexpr int DS = D / 32;          // dim steps of S^T = K Q^T
  constexpr int DB = D / 16;          // dim blocks of O^T = V^T P^T
  constexpr int KC = D / 8;           // bf16 chunks per K row
  constexpr int KS = KC + 1;          // K row stride in chunks
  constexpr int KCH = kSub * KS;      // K chunks per image
  constexpr int IMG = KCH + D * kVS;  // chunks per image
  constexpr int OST = D + 4;
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int KP = kSub * D * EB / 16;   // 16-byte global pieces of K per sub-chunk
  constexpr int VP = D * kSub * EB / 16;   // and of V
  constexpr int KPT = KP / 256, VPT = VP / 256;
  static_assert(KP % 256 == 0 && VP % 256 == 0, "pieces per thread");
  __shared__ u32x4 sm_img[2][IMG];
  // per 8-entry block of the chunk: element offsets of its first K row and
  // of its first V entry at dim 0 (-1: absent page), and E4M3 (k, v) scales
  __shared__ int64_t sm_koff[kBlkMax];
  __shared__ int64_t sm_voff[kBlkMax];
  __shared__ float2 sm_bsc[FP8 ? kBlkMax : 1];

  // chunk-major order: a short last chunk of every sequence is dispatched last
  const int npairs = a.B * a.Hkv * a.n_cgroups;
  const int wgi = blockIdx.x / npairs;
  const int x = blockIdx.x - wgi * npairs;
  const int cg = x % a.n_cgroups;
  const int bh = x / a.n_cgroups;
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const int st0 = a.start[b];
  if (!chunk_start_ok(st0, a.max_start)) return;
  const int base = draft_ctx_base(st0, a.W);
  const int nch = st0 > base ? (st0 - base + a.chunk_tokens - 1) / a.chunk_tokens : 0;
  // the block's own keys go to the last workgroup with context, or to
  // workgroup 0 when there is none
  const int wg_last = max(0, nch - 1);
  if (wgi > wg_last) return;   // past the context (uniform: before any barrier)
  const bool own_here = wgi == wg_last;
  const int p0 = base + wgi * a.chunk_tokens;
  const int p1 = max(p0, min(p0 + a.chunk_tokens, st0));   // p1 == p0: no context
  // the first position any column sees; below it cache entries may be absent
  const int lo_all = a.W > 0 ? max(0, st0 - a.W + 1) : 0;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;
  const int g4 = lane >> 4;
  const int ncols = a.T * a.G;
  const int ci = cg * kDraftGroupCols + w * 16 + col;
  const bool cok = ci < ncols;
  const int t = cok ? ci / a.G : 0;
  const int hq = hk * a.G + (cok ? ci - t * a.G : 0);
  const int lot = a.W > 0 ? max(0, st0 + t - a.W + 1) : 0;   // the column's first visible position

  const CacheView& cv = a.cache;
  const bool paged = cv.kind != MUSE_KV_RING;
  const int pt = cv.page_tokens;
  const int vstride = paged ? pt : cv.capacity;

  // The block table, filled to whole sub-chunks: blocks at or past p1 are
  // marked absent, so staging loads need no range test.  Entries below the
  // first visible position are masked where they are stored.  A block lies
  // in one page (pages hold a multiple of 16 positions, chunks start at
  // multiples of 32) and, on a ring, in one run of slots; so does a
  // 16-entry group at a multiple of 16.
  const int nblk = (p1 - p0 + kSub - 1) / kSub * (kSub / 8);
  for (int i = tid; i < nblk; i += 256) {
    const int pos = p0 + 8 * i;
    int si = -1, row = 0;
    if (pos < p1) {
      if (paged) {
        const int pi = pos / pt;
        const int page = pi < cv.max_pages ? cv.block_table[static_cast<int64_t>(b) * cv.max_pages + pi] : -1;
        if (page >= 0 && page < cv.num_pages) {
          si = page * a.Hkv + hk;
          row = pos - pi * pt;
        }
      } else {
        si = bh;
        row = pos % cv.capacity;
      }
    }
    sm_koff[i] = si >= 0 ? (static_cast<int64_t>(si) * vstride + row) * D : -1;
    sm_voff[i] = si >= 0 ? static_cast<int64_t>(si) * D * vstride + row : -1;
    if constexpr (FP8) sm_bsc[i] = si >= 0 ? float2{cv.k_scale[si], cv.v_scale[si]} : float2{0.f, 0.f};
  }

  // RoPE (sin, cos) at the block's positions, once per workgroup, in image 1
  float2* rope = reinterpret_cast<float2*>(&sm_img[1][0]);
  if (a.use_rope) {
    for (int i = tid; i < a.T * (D / 2); i += 256) {
      float sn, cs;
      rope_sincos(st0 + i / (D / 2), i % (D / 2), D, a.log2_theta, &sn, &cs);
      rope[i] = float2{sn, cs};
    }
  }
  __syncthreads();

  // q_hat of the lane's column: dims 32 ds + 8 g4 + [0, 8), which include
  // both halves of every rotate-half pair it needs (dims j and j + D/2 lie
  // DS/2 steps apart); the row's sum of squares adds the four g4 lanes
  bf16x8 qhi[DS], qlo[DS];
  {
    const uint16_t* qr = a.q + b * a.q_sb + static_cast<int64_t>(t) * a.q_st + static_cast<int64_t>(hq) * D + 8 * g4;
    float xq[DS][8];
    float ss = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 raw = cok ? *reinterpret_cast<const u32x4*>(qr + 32 * ds) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xq[ds][e] = bf16_bits_to_f32(static_cast<uint16_t>(raw[e >> 1] >> (16 * (e & 1))));
        ss += xq[ds][e] * xq[ds][e];
      }
    }
    ss += __shfl_xor(ss, 16, kWave);
    ss += __shfl_xor(ss, 32, kWave);
    const float rs = a.qscale / sqrtf(ss * (1.0f / D) + a.qk_eps);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) xq[ds][e] *= rs;
    if (a.use_rope) {
#pragma unroll
      for (int ds = 0; ds < DS / 2; ++ds)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 sc = rope[t * (D / 2) + 32 * ds + 8 * g4 + e];
          const float x0 = xq[ds][e], x1 = xq[ds + DS / 2][e];
          xq[ds][e] = x0 * sc.y - x1 * sc.x;
          xq[ds + DS / 2][e] = x1 * sc.y + x0 * sc.x;
        }
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16_t hi = static_cast<bf16_t>(xq[ds][e]);
        qhi[ds][e] = hi;
        qlo[ds][e] = static_cast<bf16_t>(xq[ds][e] - static_cast<float>(hi));
      }
  }
  __syncthreads();   // image 1 (the RoPE table) is free again

  // ---- staging: thread tid loads pieces tid + 256 i of the sub-chunk's K
  // (row-major, 16 bytes of one row each) and V (head-dim-major, 8 or 16
  // entries of one dim each), consecutive threads reading consecutive bytes
  // of a page or ring run; absent blocks read the start of the cache and
  // are zeroed at the store, as are entries outside [lo_all, p1) ----
  const uint16_t* kc = static_cast<const uint16_t*>(cv.k);
  const uint16_t* vc = static_cast<const uint16_t*>(cv.v);
  const uint8_t* kc8 = static_cast<const uint8_t*>(cv.k);
  const uint8_t* vc8 = static_cast<const uint8_t*>(cv.v);
  constexpr int KPR = D * EB / 16;         // K pieces per row
  constexpr int VPR = kSub * EB / 16;      // V pieces per dim (per sub-chunk)
  constexpr int EPV = 16 / EB;             // entries per V piece
  u32x4 stg[KPT + VPT];
  auto stage_load = [&](int s0) {
    const int blk0 = (s0 - p0) >> 3;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int p = tid + 256 * i;
      const int row = p / KPR, c = p % KPR;
      const int64_t off = max(sm_koff[blk0 + (row >> 3)], int64_t{0}) + (row & 7) * D;
      if constexpr (FP8)
        stg[i] = *reinterpret_cast<const u32x4*>(kc8 + off + 16 * c);
      else
        stg[i] = *reinterpret_cast<const u32x4*>(kc + off + 8 * c);
    }
    // the V pieces of a thread share one block (c is tid % VPR)
    const int cv0 = tid % VPR;
    const int64_t vb = max(sm_voff[blk0 + cv0 * EPV / 8], int64_t{0});
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int d = vdim<FP8>((tid + 256 * i) / VPR);
      if constexpr (FP8)
        stg[KPT + i] = *reinterpret_cast<const u32x4*>(vc8 + vb + static_cast<int64_t>(d) * vstride);
      else
        stg[KPT + i] = *reinterpret_cast<const u32x4*>(vc + vb + static_cast<int64_t>(d) * vstride);
    }
  };
  // 16-bit halves of a V chunk kept for entries e0 .. e0 + 7 in [lo, hi)
  auto keep8 = [](int e0, int lo, int hi) {
    u32x4 mk;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const int e = e0 + 2 * wd;
      mk[wd] = ((e >= lo && e < hi) ? 0xffffu : 0u) | ((e + 1 >= lo && e + 1 < hi) ? 0xffff0000u : 0u);
    }
    return mk;
  };
  // every block of the sub-chunk present and every entry in [lo_all, p1):
  // nothing to mask (the same answer in every lane)
  auto all_in = [&](int s0) {
    const bool pres = sm_koff[((s0 - p0) >> 3) + (lane & 7)] >= 0;
    return s0 >= lo_all && s0 + kSub <= p1 && __builtin_amdgcn_ballot_w64(!pres) == 0;
  };
  auto stage_store = [&](int buf, int s0) {
    u32x4* img = sm_img[buf];
    const int blk0 = (s0 - p0) >> 3;
    const bool full = all_in(s0);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int p = tid + 256 * i;
      const int row = p / KPR, c = p % KPR;
      const int e = s0 + row;
      const bool ok = full || (e >= lo_all && e < p1 && sm_koff[blk0 + (row >> 3)] >= 0);
      const int at = kperm(row) * KS;
      if constexpr (FP8) {
        u32x4 lo, hi;
        e4m3x16_to_bf16(stg[i], lo, hi);
        img[at + 2 * c] = ok ? lo : u32x4{0, 0, 0, 0};
        img[at + 2 * c + 1] = ok ? hi : u32x4{0, 0, 0, 0};
      } else {
        img[at + c] = ok ? stg[i] : u32x4{0, 0, 0, 0};
      }
    }
    const int c = tid % VPR;
    const int e0 = c * EPV;
    u32x4 m0 = {~0u, ~0u, ~0u, ~0u}, m1 = m0;
    if (!full) {
      const bool bok = sm_koff[blk0 + (e0 >> 3)] >= 0;
      m0 = bok ? keep8(s0 + e0, lo_all, p1) : u32x4{0, 0, 0, 0};
      m1 = bok ? keep8(s0 + e0 + 8, lo_all, p1) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int d = vdim<FP8>((tid + 256 * i) / VPR);
      if constexpr (FP8) {
        u32x4 lo, hi;
        e4m3x16_to_bf16(stg[KPT + i], lo, hi);
        img[KCH + d * kVS + 2 * c] = lo & m0;
        img[KCH + d * kVS + 2 * c + 1] = hi & m1;
      } else {
        img[KCH + d * kVS + c] = stg[KPT + i] & m0;
      }
    }
  };

  float m = kNeg, lsum = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // largest first visible position over the workgroup's columns: a
  // sub-chunk from there to p1 with every block present needs no masks
  int lot_max = cok ? lot : 0;
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) lot_max = max(lot_max, __shfl_xor(lot_max, msk, kWave));
  lot_max = __builtin_amdgcn_readfirstlane(lot_max);

  // one sub-chunk from image buf: entries s0 + [0, 64) of the context, or
  // the block's own keys (own: K as hi in image 0 plus lo in image 1's K
  // rows, visible below position hi_own)
  auto compute = [&](int buf, int s0, bool own, int hi_own) {
    const u32x4* K = sm_img[buf];
    const u32x4* Klo = sm_img[1];
    const u32x4* V = sm_img[buf] + KCH;
    const int blk0 = (s0 - p0) >> 3;
    // past every column's first visible position, all blocks present: no masks
    const bool inner = !own && s0 >= lot_max && all_in(s0);
    const int ehi = own ? hi_own : p1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // logits of entries s0 + 32 h + 8 g4 + 4 kt + i, i < 4: block 4 h + g4
      const int blk = own ? 0 : blk0 + 4 * h + g4;   // the own keys have no block table
      const bool bok = own || sm_koff[blk] >= 0;
      float ks = 1.f, vs = 1.f;
      if constexpr (FP8) {
        if (!own) {
          const float2 sc = sm_bsc[blk];
          ks = sc.x;
          vs = sc.y;
        }
      }
      float sv[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          // image row 32h + 16kt + col holds entry 32h + 8(col >> 2) + 4kt + (col & 3)
          const int ch = (32 * h + 16 * kt + col) * KS + 4 * ds + g4;
          const bf16x8 kf = __builtin_bit_cast(bf16x8, K[ch]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qhi[ds], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[ds], acc, 0, 0, 0);
          if (own) {
            const bf16x8 kl = __builtin_bit_cast(bf16x8, Klo[ch]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qhi[ds], acc, 0, 0, 0);
          }
        }
        if (inner) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[kt][i] = cok ? acc[i] * ks : kNeg;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = s0 + 32 * h + 8 * g4 + 4 * kt + i;
            const bool vis = cok && bok && e >= lot && e < ehi;
            sv[kt][i] = vis ? acc[i] * ks : kNeg;
          }
        }
      }
      float tmax = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                         fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
      if (__builtin_amdgcn_ballot_w64(tmax > m + kSlack) != 0) {
        // the four lanes of a column share its maximum
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const float mnew = fmaxf(m, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      bf16x8 phi, plo;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = sv[kt][i] > kNeg ? __builtin_amdgcn_exp2f(sv[kt][i] - m) : 0.f;
          psum += pw;
          const float pv = pw * vs;
          const bf16_t hi = static_cast<bf16_t>(pv);
          phi[4 * kt + i] = hi;
          plo[4 * kt + i] = static_cast<bf16_t>(pv - static_cast<float>(hi));
        }
      lsum += psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, V[(16 * db + col) * kVS + 4 * h + g4]);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi, o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo, o[db], 0, 0, 0);
      }
    }
  };

  // ---- context: image j % 2 is computed while sub-chunk j + 1's loads are
  // in flight; they are stored into the other image afterwards ----
  const int nsub = (p1 - p0 + kSub - 1) / kSub;
  if (nsub > 0) {
    stage_load(p0);
    stage_store(0, p0);
    if (nsub > 1) stage_load(p0 + kSub);
    for (int j = 0; j < nsub; ++j) {
      __syncthreads();   // image j % 2 is complete, image (j + 1) % 2 is no longer read
      compute(j & 1, p0 + kSub * j, false, 0);
      if (j + 1 < nsub) {
        stage_store((j + 1) & 1, p0 + kSub * (j + 1));
        if (j + 2 < nsub) stage_load(p0 + kSub * (j + 2));
      }
    }
  }

  // ---- the block's own keys: k_hat (normalized, rotated, fp32) as bf16 hi
  // (image 0) + lo (image 1's K rows), v transposed into image 0's V part;
  // rows past T are zero and masked ----
  if (own_here) {
    __syncthreads();   // the images are no longer read
    u32x4* img0 = sm_img[0];
    u32x4* img1 = sm_img[1];
    for (int i = tid; i < KCH; i += 256) {
      img0[i] = u32x4{0, 0, 0, 0};
      img1[i] = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
    {
      constexpr int LPR = D / 2;
      constexpr int RPI = 256 / LPR;     // rows per pass
      const int j = tid % LPR;
      for (int tt0 = 0; tt0 < a.T; tt0 += RPI) {   // uniform: the row sums stay convergent
        const int tt = tt0 + tid / LPR;
        const bool valid = tt < a.T;
        float x0 = 0.f, x1 = 0.f;
        if (valid) {
          const uint16_t* kr = a.k + b * a.k_sb + static_cast<int64_t>(tt) * a.k_st + static_cast<int64_t>(hk) * D;
          x0 = bf16_bits_to_f32(kr[j]);
          x1 = bf16_bits_to_f32(kr[j + D / 2]);
        }
        const float ss = group_sum<LPR>(x0 * x0 + x1 * x1);
        const float r = 1.0f / sqrtf(ss * (1.0f / D) + a.qk_eps);
        x0 *= r;
        x1 *= r;
        float y0 = x0, y1 = x1;
        if (a.use_rope && valid) {
          float sn, cs;
          rope_sincos(st0 + tt, j, D, a.log2_theta, &sn, &cs);
          y0 = x0 * cs - x1 * sn;
          y1 = x1 * cs + x0 * sn;
        }
        if (valid) {
          bf16_t* k0 = reinterpret_cast<bf16_t*>(img0);
          bf16_t* k1 = reinterpret_cast<bf16_t*>(img1);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int dd = j + hh * (D / 2);
            const float y = hh ? y1 : y0;
            const int at = (kperm(tt) * KS + (dd >> 3)) * 8 + (dd & 7);
            const bf16_t yh = static_cast<bf16_t>(y);
            k0[at] = yh;
            k1[at] = static_cast<bf16_t>(y - static_cast<float>(yh));
          }
        }
      }
    }
    // V: chunk (d, c) holds entries 8c .. 8c + 7 of dim d
    for (int i = tid; i < D * 8; i += 256) {
      const int d = i / 8, c = i % 8;
      u32x4 ch;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        uint32_t pr = 0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int tt = 8 * c + 2 * wd + hh;
          const uint32_t bits =
              tt < a.T ? a.v[b * a.v_sb + static_cast<int64_t>(tt) * a.v_st + static_cast<int64_t>(hk) * D + d] : 0u;
          pr |= bits << (16 * hh);
        }
        ch[wd] = pr;
      }
      img0[KCH + d * kVS + c] = ch;
    }
    __syncthreads();
    // visible: |t - t'| < W (every key of the block when W = 0)
    const int hi_own = a.W > 0 ? min(st0 + a.T, st0 + t + a.W) : st0 + a.T;
    compute(0, st0, true, hi_own);
  }

  // ---- partial of the lane's column ----
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  float* prow = a.part + ((static_cast<int64_t>(x) * a.n_wg + wgi) * kDraftGroupCols + w * 16 + col) * OST;
#pragma unroll
  for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(prow + 16 * db + 4 * g4) = o[db];
  if (g4 == 0) {
    prow[D] = m;
    prow[D + 1] = lsum;
  }
}

// ---------------------------------------------------------------------------
// 2. combine + epilogue: one wave per (sequence, token, query head), four
// heads per workgroup; lane l holds output dims l (and l + 64 at D = 128).
// Every load is issued before the arithmetic that waits on one: the gate
// and the first kPre partials (clamped indices; the values of absent ones
// are replaced by zeros, as the workspace there holds whatever was left in
// it).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void draft_combine_kernel(DraftArgs a) {
  constexpr int PL = D / kWave;  // output dims per lane
  constexpr int OST = D + 4;
  constexpr int kPre = 4;
  const int Hq = a.Hkv * a.G;
  const int hpb = (Hq + kWavesDraft - 1) / kWavesDraft;
  int x = blockIdx.x;
  const int hb = x % hpb;
  x /= hpb;
  const int t = x % a.T;
  const int b = x / a.T;
  const int hq = hb * kWavesDraft + (threadIdx.x >> 6);
  if (hq >= Hq) return;  // no barriers below
  const int lane = threadIdx.x & 63;
  uint16_t* orow = a.out + b * a.o_sb + static_cast<int64_t>(t) * a.o_st + static_cast<int64_t>(hq) * D;
  const int st0 = a.start[b];
  if (!chunk_start_ok(st0, a.max_start)) {
#pragma unroll
    for (int e = 0; e < PL; ++e) orow[lane + kWave * e] = 0;
    return;
  }
  const int base = draft_ctx_base(st0, a.W);
  const int nch = st0 > base ? (st0 - base + a.chunk_tokens - 1) / a.chunk_tokens : 0;
  const int nparts = max(nch, 1);   // partials written (the block's own keys are in the last one)
  const int hk = hq / a.G;
  const int ci = t * a.G + (hq - hk * a.G);
  const int64_t grp = (static_cast<int64_t>(b) * a.Hkv + hk) * a.n_cgroups + ci / kDraftGroupCols;
  const float* part0 = a.part + (grp * a.n_wg * kDraftGroupCols + ci % kDraftGroupCols) * OST;
  const int64_t pstride = static_cast<int64_t>(kDraftGroupCols) * OST;

  float gv[PL];
  {
    const uint16_t* gr = a.gate + b * a.g_sb + static_cast<int64_t>(t) * a.g_st + static_cast<int64_t>(hq) * D;
#pragma unroll
    for (int e = 0; e < PL; ++e) gv[e] = bf16_bits_to_f32(gr[lane + kWave * e]);
  }
  float pm[kPre], pl[kPre], po[kPre][PL];
#pragma unroll
  for (int c = 0; c < kPre; ++c) {
    const float* pc = part0 + min(c, nparts - 1) * pstride;
    pm[c] = pc[D];
    pl[c] = pc[D + 1];
#pragma unroll
    for (int e = 0; e < PL; ++e) po[c][e] = pc[lane + kWave * e];
    if (c >= nparts) {   // a repeat of the last partial: weight zero
      pm[c] = kNeg;
      pl[c] = 0.f;
#pragma unroll
      for (int e = 0; e < PL; ++e) po[c][e] = 0.f;
    }
  }
  float mx = kNeg;
#pragma unroll
  for (int c = 0; c < kPre; ++c) mx = fmaxf(mx, pm[c]);
  for (int c = kPre; c < nparts; ++c) mx = fmaxf(mx, part0[c * pstride + D]);
  // mx is finite: token t sees its own key, in the last partial

  float l = 0.f, acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
  // a column that saw nothing of a chunk has max kNeg there: weight 0
#pragma unroll
  for (int c = 0; c < kPre; ++c) {
    const float wgt = __builtin_amdgcn_exp2f(pm[c] - mx);
    l += wgt * pl[c];
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] += wgt * po[c][e];
  }
  for (int c = kPre; c < nparts; ++c) {
    const float* pc = part0 + c * pstride;
    const float wgt = __builtin_amdgcn_exp2f(pc[D] - mx);
    l += wgt * pc[D + 1];
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] += wgt * pc[lane + kWave * e];
  }
  const float inv = 1.0f / l;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    acc[e] *= inv;
    ss += acc[e] * acc[e];
  }
  float rsn = 1.0f;
  if (a.out_norm) rsn = 1.0f / sqrtf(wave_sum(ss) * (1.0f / D) + a.out_eps);
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    const float sg = 1.0f / (1.0f + __expf(-gv[e]));
    orow[lane + kWave * e] = f32_to_bf16_bits(acc[e] * rsn * sg);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {
template <int D>
hipError_t launch_draft_d(const DraftArgs& a, hipStream_t st) {
  const int Hq = a.Hkv * a.G;
  const unsigned g1 = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * a.n_cgroups * a.n_wg);
  if (a.cache.fp8)
    hipLaunchKernelGGL((draft_split_kernel<D, true>), dim3(g1), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((draft_split_kernel<D, false>), dim3(g1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t g2 = static_cast<int64_t>(a.B) * a.T * ((Hq + kWavesDraft - 1) / kWavesDraft);
  hipLaunchKernelGGL((draft_combine_kernel<D>), dim3(static_cast<unsigned>(g2)), dim3(256), 0, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_draft(int d, const DraftArgs& a, hipStream_t st) {
  return d == 64 ? launch_draft_d<64>(a, st) : launch_draft_d<128>(a, st);
}

}  // namespace muse
