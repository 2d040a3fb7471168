// Prefill attention: grouped-query attention with the weightless QK-norm
// prologue for the queries fused into the load, a max-free exponential
// softmax, MFMA contractions, and the output norm + sigmoid gate epilogue.
//
// What it computes (Muse Spark Open deep dive):
//   section 3.2: q_hat = s * q / sqrt(mean(q^2) + eps), logits q_hat . k_hat / sqrt(D);
//   section 3.4: RoPE on local layers, causal window i - W < j <= i;
//   section 3.1: query head h reads KV head floor(h / G);
//   section 3.3: Spark per-head output RMS norm, then y = o * sigmoid(g).
//
// Design for gfx950:
//   * One workgroup owns BQ consecutive tokens of one (sequence, KV head) and
//     all G query heads of that group: 256 query rows = (token, head) pairs,
//     so each K/V tile staged in LDS feeds every head of the group.
//   * Logits are bounded: with unit-RMS q_hat/s and k_hat, |logit| <=
//     s * sqrt(D) = 43.784 (section 3.2 logit equation), i.e. <= 63.2 in
//     log2 units.  exp2 of that range, and sums of 2^20 such terms, stay
//     inside fp32 and bf16 range, so the softmax needs no running maximum and
//     no rescaling of the accumulator: p = exp2(logit * log2 e) directly.
//   * S^T = K * Q^T with v_mfma_f32_32x32x16_f16 (q_hat, k_hat in fp16: the
//     normalized operands are bounded by sqrt(D) * s, and fp16 keeps 3 more
//     mantissa bits than bf16); O^T = V^T * P^T with v_mfma_f32_32x32x16_bf16.
//     The S^T accumulator layout is exactly the P^T operand layout of the
//     second MFMA, so P never leaves registers.
//   * Tiles are copied verbatim from the pre-swizzled workspace into a
//     three-buffer LDS ring (two tiles resident, the next in flight); only
//     tiles crossing the causal diagonal or the window start are masked, and
//     a wave skips edge tiles it cannot see.  Between the edges the loop is
//     software-pipelined: the logits of the next half-tile go to the matrix
//     cores while the exponentials of the current one run on the vector ALUs.
//   * Launch order: heaviest query blocks first (causal work grows with the
//     block index), and groups of 8 consecutive query blocks of one KV head
//     land on one XCD so they share K/V tiles in that XCD's L2.
#include "kernels.h"

namespace muse {

constexpr int kQBlockGroup = 8;

template <int D, int G, int NW, int MB>
struct PrefillCfg {
  static constexpr int ROWS = NW * MB * 32;
  static constexpr int BQ = ROWS / G;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int THREADS = NW * 64;
  static constexpr int KCH = 8 * D;  // 16-byte chunks of one K (or V) tile
  static constexpr int CPT = KCH / THREADS;
  static_assert(32 % G == 0 || G == 32, "a 32-row block must hold whole tokens");
  static_assert(KCH % THREADS == 0, "tile copy must divide evenly");
};

template <int D, int G, int NW, int MB>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D, G, NW, MB>;
  constexpr int NBUF = 3;
  __shared__ u32x4 smem[NBUF][2 * C::KCH];

  // ---- workgroup -> (sequence, KV head, query block) ----
  const int nblk = gridDim.x;
  const int raw = blockIdx.x;
  constexpr int QC = kQBlockGroup;
  int L = raw;
  const int full_groups = (nblk / (8 * QC)) * (8 * QC);
  if (raw < full_groups) {
    const int slot = raw >> 3, xcd = raw & 7;
    L = (slot / QC) * (8 * QC) + xcd * QC + (slot % QC);
  }
  const int per = a.batch_heads * QC;
  const int qbc = L / per;
  const int rem = L - qbc * per;
  const int bh = rem / QC;
  const int qi = rem - bh * QC;
  const int qb = a.n_qblocks_pad - 1 - (qbc * QC + qi);
  if (qb >= a.n_qblocks) return;  // padding block: exits before any barrier
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const int t0 = qb * C::BQ;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // ---- queries: load, weightless RMS norm, scale, RoPE, fp16 operands ----
  half8 qf[MB][C::KS];
  int tq[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = (w * MB + mb) * 32 + l32;
    const int t = t0 + r / G;
    const int hq = hk * G + (r % G);
    tq[mb] = t;
    float x[C::KS][8];
    const bool valid = t < a.T;
    const uint16_t* qp = a.q + b * a.q_sb + static_cast<int64_t>(t) * a.q_st + static_cast<int64_t>(hq) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 wv = {0, 0, 0, 0};
      if (valid) wv = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      unpack_bf16x8(wv, x[ks]);
    }
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
    ss += __shfl_xor(ss, 32, kWave);
    const float rs = a.qscale * __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.qk_eps);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[ks][e] *= rs;
    if (a.rope && valid) {
      const float2* rt = a.rope + ((a.rope_batched ? static_cast<int64_t>(b) * a.T : 0) + t) * (D / 2) + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < C::KS / 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = rt[16 * ks + e];
          const float x0 = x[ks][e], x1 = x[ks + C::KS / 2][e];
          x[ks][e] = x0 * cs.x - x1 * cs.y;
          x[ks + C::KS / 2][e] = x1 * cs.x + x0 * cs.y;
        }
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[mb][ks][e] = static_cast<half_t>(x[ks][e]);
  }

  // ---- key range: masked edge tiles and the unmasked middle ----
  const int tlast = min(t0 + C::BQ, a.T) - 1;      // last real token of the block
  const int klo = a.W > 0 ? max(0, t0 - a.W + 1) : 0;
  const int tile_lo = klo / kKeyTile;
  const int tile_hi = tlast / kKeyTile;
  // tiles fully visible to every token of the block: k0 + 63 <= t0 and k0 > tlast - W
  int mid_lo = tile_lo;
  if (a.W > 0) {
    const int first_full = tlast - a.W + 1;                 // need k0 >= first_full
    mid_lo = max(tile_lo, (max(first_full, 0) + kKeyTile - 1) / kKeyTile);
  }
  const int mid_hi = min((t0 + 1) / kKeyTile, tile_hi + 1);  // need k0 + 63 <= t0
  const int m_lo = min(mid_lo, mid_hi);
  const int m_hi = max(mid_hi, m_lo);
  const int tw0 = t0 + (w * MB * 32) / G;
  const int tw1 = t0 + ((w + 1) * MB * 32 - 1) / G;

  // per-lane visible range of each row block: key in [lo_t, lo_t + span]
  int lo_t[MB], span[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    lo_t[mb] = a.W > 0 ? max(0, tq[mb] - a.W + 1) : 0;
    span[mb] = tq[mb] - lo_t[mb];
  }

  const u32x4* ksrc = reinterpret_cast<const u32x4*>(a.khat) + static_cast<int64_t>(bh) * a.n_tiles * C::KCH;
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(a.vt) + static_cast<int64_t>(bh) * a.n_tiles * C::KCH;

  f32x16 o[MB][C::DB];
  float lsum[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    lsum[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mb][db][i] = 0.f;
  }

  // ---- tile staging: three LDS buffers, tiles i and i+1 resident while
  // tile i+2 is in flight in registers ----
  u32x4 pre[2 * C::CPT];
  auto gload = [&](int tile) {
    const int64_t base = static_cast<int64_t>(tile) * C::KCH;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      pre[i] = ksrc[base + tid + i * C::THREADS];
      pre[C::CPT + i] = vsrc[base + tid + i * C::THREADS];
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      smem[buf][tid + i * C::THREADS] = pre[i];
      smem[buf][C::KCH + tid + i * C::THREADS] = pre[C::CPT + i];
    }
  };
  // after computing tile `tile`: stage tile+2, fetch tile+3, barrier
  auto advance = [&](int tile) {
    const int rel = tile - tile_lo;
    if (tile + 2 <= tile_hi) sstore((rel + 2) % NBUF);
    if (tile + 3 <= tile_hi) gload(tile + 3);
    __syncthreads();
  };

  bf16x2 ones;
  ones[0] = static_cast<bf16_t>(1.0f);
  ones[1] = static_cast<bf16_t>(1.0f);

  auto qk = [&](int tile, int kb, f32x16* s) {
    const half_t* Ks = reinterpret_cast<const half_t*>(&smem[(tile - tile_lo) % NBUF][0]);
    const int krow = 32 * kb + l32;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const half8 kf = *reinterpret_cast<const half8*>(Ks + krow * D + k_chunk_swizzle<D>(2 * ks + h2, krow) * 8);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[mb][ks], s[mb], 0, 0, 0);
    }
  };
  // p = exp2(logit): logits are bounded by 63.2 in log2 units (no max needed)
  auto softmax = [&](const f32x16* s, bf16x8 (*p)[2], bool masked, int k0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int kbase = k0 + 4 * h2 - lo_t[mb];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[mb][i];
        if (masked) {
          const int off = 8 * (i >> 2) + (i & 3);
          x = static_cast<unsigned>(kbase + off) <= static_cast<unsigned>(span[mb]) ? x : -INFINITY;
        }
        p[mb][i >> 3][i & 7] = static_cast<bf16_t>(__builtin_amdgcn_exp2f(x));
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x2 pr;
          pr[0] = p[mb][st][2 * j];
          pr[1] = p[mb][st][2 * j + 1];
          lsum[mb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum[mb], false);
        }
    }
  };
  auto pv = [&](int tile, int kb, bf16x8 (*p)[2]) {
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(&smem[(tile - tile_lo) % NBUF][C::KCH]);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int dim = 32 * db + l32;
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(Vs + dim * kKeyTile + v_chunk_swizzle(4 * kb + 2 * st + h2, dim) * 8);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          o[mb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[mb][st], o[mb][db], 0, 0, 0);
      }
  };
  // one edge tile, masked per element, skipped by waves that see none of it
  auto edge_tile = [&](int tile) {
    const int k0 = tile * kKeyTile;
    const bool any = (k0 <= tw1) && (a.W == 0 || k0 + kKeyTile - 1 > tw0 - a.W);
    if (any) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s[MB];
        bf16x8 p[MB][2];
        qk(tile, kb, s);
        softmax(s, p, true, k0 + 32 * kb);
        pv(tile, kb, p);
      }
    }
    advance(tile);
  };

  // prologue: tiles 0 and 1 of the range into LDS, tile 2 in flight
  gload(tile_lo);
  sstore(0);
  if (tile_lo + 1 <= tile_hi) {
    gload(tile_lo + 1);
    sstore(1);
  }
  if (tile_lo + 2 <= tile_hi) gload(tile_lo + 2);
  __syncthreads();

  int tile = tile_lo;
  for (; tile < m_lo; ++tile) edge_tile(tile);
  if (tile < m_hi) {
    // software-pipelined middle: the logits of the next half-tile are
    // computed on the matrix cores while the exponentials of the current one
    // run on the vector ALUs.
    f32x16 s0[MB], s1[MB];
    bf16x8 p[MB][2];
    qk(tile, 0, s0);
    for (; tile < m_hi - 1; ++tile) {
      qk(tile, 1, s1);
      softmax(s0, p, false, 0);
      pv(tile, 0, p);
      qk(tile + 1, 0, s0);
      softmax(s1, p, false, 0);
      pv(tile, 1, p);
      advance(tile);
    }
    qk(tile, 1, s1);
    softmax(s0, p, false, 0);
    pv(tile, 0, p);
    softmax(s1, p, false, 0);
    pv(tile, 1, p);
    advance(tile);
    ++tile;
  }
  for (; tile <= tile_hi; ++tile) edge_tile(tile);

  // ---- epilogue: 1/sum, per-head output norm, sigmoid gate, bf16 store ----
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const float ltot = lsum[mb] + __shfl_xor(lsum[mb], 32, kWave);
    const float inv = __builtin_amdgcn_rcpf(ltot);
    float ss = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o[mb][db][i] *= inv;
        ss += o[mb][db][i] * o[mb][db][i];
      }
    float rsn = 1.0f;
    if (a.out_norm) {
      ss += __shfl_xor(ss, 32, kWave);
      rsn = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.out_eps);
    }
    const int t = tq[mb];
    if (t < a.T) {
      const int r = (w * MB + mb) * 32 + l32;
      const int hq = hk * G + (r % G);
      const uint16_t* gp = a.gate + b * a.g_sb + static_cast<int64_t>(t) * a.g_st + static_cast<int64_t>(hq) * D;
      uint16_t* op = a.out + b * a.o_sb + static_cast<int64_t>(t) * a.o_st + static_cast<int64_t>(hq) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int d0 = 32 * db + 8 * grp + 4 * h2;
          const u32x2 gw = *reinterpret_cast<const u32x2*>(gp + d0);
          float g[4] = {__uint_as_float(gw[0] << 16), __uint_as_float(gw[0] & 0xffff0000u),
                        __uint_as_float(gw[1] << 16), __uint_as_float(gw[1] & 0xffff0000u)};
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g[e]));
            y[e] = o[mb][db][4 * grp + e] * rsn * sg;
          }
          *reinterpret_cast<u32x2*>(op + d0) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {
constexpr int kWaves = 8;
constexpr int kRowBlocks = 1;

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a, hipStream_t st) {
  using C = PrefillCfg<D, G, kWaves, kRowBlocks>;
  const unsigned grid = static_cast<unsigned>(a.n_qblocks_pad) * static_cast<unsigned>(a.batch_heads);
  hipLaunchKernelGGL((prefill_kernel<D, G, kWaves, kRowBlocks>), dim3(grid), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int g, const PrefillArgs& a, hipStream_t st) {
  switch (g) {
    case 1: return launch_dg<D, 1>(a, st);
    case 2: return launch_dg<D, 2>(a, st);
    case 4: return launch_dg<D, 4>(a, st);
    case 8: return launch_dg<D, 8>(a, st);
    case 16: return launch_dg<D, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

int prefill_rows_per_block(int, int) { return kWaves * kRowBlocks * 32; }

int prefill_qblock_group() { return kQBlockGroup; }

hipError_t launch_prefill(int d, int g, const PrefillArgs& a, hipStream_t st) {
  return d == 64 ? launch_d<64>(g, a, st) : launch_d<128>(g, a, st);
}

}  // namespace muse
