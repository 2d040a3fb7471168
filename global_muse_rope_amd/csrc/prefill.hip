// Prefill attention: grouped-query attention with the weightless QK-norm
// prologue for the queries fused into the load, a max-free exponential
// softmax, MFMA contractions, and the output norm + sigmoid gate epilogue.
//
// What it computes (Muse Spark Open deep dive):
//   section 3.2: q_hat = s * q / sqrt(mean(q^2) + eps), logits q_hat . k_hat / sqrt(D);
//   section 3.4: RoPE on local layers, causal window i - W < j <= i;
//   section 8.2: a drafter's block sees the two-sided window |i - j| < W;
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
//     Cached history (chunked prefill, drafter blocks) is read as stored,
//     so its keys need not have unit RMS: the block's bound then scales
//     with the largest cached-key RMS of its range, and logits are shifted
//     by a constant per block where that bound passes kLogitCap.
//   * S^T = K * Q^T with v_mfma_f32_32x32x16_f16 (q_hat, k_hat in fp16: the
//     normalized operands are bounded by sqrt(D) * s, and fp16 keeps 3 more
//     mantissa bits than bf16); O^T = V^T * P^T with v_mfma_f32_32x32x16_bf16.
//     The S^T accumulator layout is exactly the P^T operand layout of the
//     second MFMA, so P never leaves registers.
//   * Tiles are copied verbatim from the pre-swizzled workspace into a
//     four-buffer LDS ring (three tiles resident, the next in flight); a
//     block visits only the tiles its rows can see, and only the first and
//     last of them (crossing the diagonal or a window edge) are masked.  The
//     loop is software-pipelined: the logits of the next half-tile go to the
//     matrix cores while the exponentials of the current one run on the
//     vector ALUs.
//   * Launch order.  Global layers: heaviest query blocks first (causal work
//     grows with the block index), and groups of 8 consecutive query blocks
//     of one KV head land on one XCD so they share K/V tiles in its L2.
//     Local layers (uniform work): each XCD walks one contiguous range of
//     query blocks, so the 2048-key window's tiles stay in that XCD's L2.
//     Launches with fewer query blocks than CUs (a short chunk, a drafter's
//     block) split each block's tile range over several workgroups, and
//     prefill_combine_kernel adds the pieces.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace muse {

constexpr int kQBlockGroup = 8;
// LDS fragment queue depth (fragments in flight per wave) per head width.
// Head width 64 keeps the register count low enough for two workgroups per CU.
constexpr int kFragQueueD128 = 8;
constexpr int kFragQueueD64 = 2;
// s_waitcnt immediate that waits for vmcnt(0) only (expcnt and lgkmcnt at
// their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

// One wave's share of a tile copy: R consecutive rounds of 64 lanes x 16
// bytes (1 KB each) from global memory straight into LDS
// (global_load_lds_dwordx4).  The LDS address comes from M0, uniform over the
// wave, and the global address is a scalar base plus a per-lane offset; the
// instruction's immediate offset advances the global and the LDS address
// alike, so all rounds share one base, one lane offset and one M0 value (one
// M0 write per tile instead of one per round, and no per-round address
// arithmetic in the tile loop).
// The copies are counted by VM_CNT alone: the kernel waits for them with an
// explicit vmcnt(0) before the barrier that publishes the tile.  Issued
// through the builtin, the compiler treats each as a flat access that may
// also touch LDS and, while one is in flight, turns every wait on an LDS
// fragment read into lgkmcnt(0), draining the fragment queue twice per
// half-tile.  Written as instructions of their own the compiler keeps its
// exact lgkmcnt(7) waits; the statement has no register outputs, and its
// memory clobber keeps LDS accesses from moving across it.
template <int R>
__device__ __forceinline__ void dma_wave_share(const u32x4* wave_src, uint32_t lane_off, void* lds_wave_base) {
  static_assert(R == 2 || R == 4, "1 KB rounds within the 4 KB immediate offset range");
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_wave_base)));
  const uint64_t p = reinterpret_cast<uint64_t>(wave_src);
  // readfirstlane returns int: each half goes through uint32_t, so the low
  // half is zero-extended, not sign-extended, into the 64-bit address
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32)));
  const uint64_t sp = (static_cast<uint64_t>(hi) << 32) | lo;
  if constexpr (R == 4)
    asm volatile(
        "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:3072" ::"v"(lane_off),
        "s"(sp), "s"(m0)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:1024" ::"v"(lane_off),
        "s"(sp), "s"(m0)
        : "memory", "m0");
}

template <int D, int G, int NW, int MB>
struct PrefillCfg {
  static constexpr int ROWS = NW * MB * 32;
  static constexpr int BQ = ROWS / G;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int THREADS = NW * 64;
  static_assert(32 % G == 0 || G == 32, "a 32-row block must hold whole tokens");
};

// SKIP: waves whose columns all lie past the last query row skip their
// matrix and vector work (launches whose sequences are shorter than a block).
// HMODE: 0, no cached history (whole-sequence prefill): the logit
// accumulators start at the constant 0.  Cached history read as stored
// (chunked prefill, drafter blocks) brings a per-block logit bound read from
// tile_ms, and each such launch is a pair: HMODE 1 computes the blocks whose
// bound needs no shift (constant 0 start) and skips the others, HMODE 2 the
// blocks that need one (the accumulators start at the shift) and skips the
// rest.  One copy of the tile loop per instance keeps the register count
// (and occupancy) of the common case.
template <int D, int G, int NW, int MB, bool SKIP, int HMODE>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D, G, NW, MB>;
  using TL = TileLayout<D>;
  constexpr int NBUF = 4;
  // four tile buffers; the epilogue stages its fp32 outputs (padded columns)
  // in the same memory
  constexpr int OROW = D + 4;  // floats per staged column
  constexpr int STAGE_CHUNKS = NW * MB * 32 * OROW / 4;
  constexpr int SMEM_CHUNKS = NBUF * TL::CHUNKS > STAGE_CHUNKS ? NBUF * TL::CHUNKS : STAGE_CHUNKS;
  __shared__ u32x4 smem[SMEM_CHUNKS];
  auto tile_buf = [&](int buf) -> u32x4* { return smem + buf * TL::CHUNKS; };


  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // ---- workgroups -> (sequence, KV head, query block) ----
  // Workgroups are dealt to the 8 XCDs round-robin (blockIdx mod 8), and each
  // XCD runs its share in increasing blockIdx order.
  //   Local layer (uniform work per block): a persistent grid; XCD x owns one
  //   contiguous range of logical blocks and its K workgroups walk it with
  //   stride K, so the XCD works on K consecutive query blocks at a time and
  //   the window's tiles stay in its L2.
  //   Global layer: one block per workgroup, heaviest (latest) query blocks
  //   first, groups of QC consecutive blocks of one KV head on one XCD.
  const int nlog = a.n_qblocks_pad * a.batch_heads;  // a multiple of 8
  constexpr int QC = kQBlockGroup;
  //   Key split: one (query block, key piece) per workgroup, pieces of a
  //   block on consecutive workgroups.
  // (head width 64 already fits two workgroups per CU, which overlap each
  // other's block starts; the persistent loop's registers would cost that)
  const bool split = a.nsplit > 1;
  const bool persistent = D == 128 && a.W > 0 && !split;
  int lx_first, lx_end, lx_step;
  if (persistent) {
    const int per = nlog >> 3;
    const int xcd = blockIdx.x & 7;
    lx_first = xcd * per + (blockIdx.x >> 3);
    lx_end = (xcd + 1) * per;
    lx_step = gridDim.x >> 3;
  } else {
    lx_first = blockIdx.x;
    lx_end = blockIdx.x + 1;
    lx_step = 1;
  }
  auto block_of = [&](int lx, int& bh, int& qb) {
    if (split) {
      const int ql = lx / a.nsplit;
      bh = ql / a.n_qblocks;
      qb = ql - bh * a.n_qblocks;
    } else if (persistent) {
      bh = lx / a.n_qblocks_pad;
      qb = lx - bh * a.n_qblocks_pad;
    } else {
      int L = lx;
      const int full_groups = (nlog / (8 * QC)) * (8 * QC);
      if (lx < full_groups) {
        const int slot = lx >> 3, xcd = lx & 7;
        L = (slot / QC) * (8 * QC) + xcd * QC + (slot % QC);
      }
      const int per = a.batch_heads * QC;
      const int qbc = L / per;
      const int rem = L - qbc * per;
      bh = rem / QC;
      const int qi = rem - bh * QC;
      qb = a.n_qblocks_pad - 1 - (qbc * QC + qi);
    }
  };

  // Raw query words (and their rotation's (cos, sin) rows) of one query
  // block.  The persistent loop loads the next block's while the current
  // block's epilogue runs, so their latency is off the next prologue.
  u32x4 qraw[MB][C::KS];
  float2 traw[MB][C::KS / 2][8];
  int qraw_lx = -1;  // the block whose rows qraw holds (uniform)
  // Every call writes all of qraw and traw (zeros where nothing is loaded),
  // so their registers are free again during the tile loop.
  auto load_q = [&](int lx_q, bool any) {
    int bh_q = 0, qb_q = 0;
    if (any) block_of(lx_q, bh_q, qb_q);
    const bool blk = any && qb_q < a.n_qblocks;  // not a padding block
    const int b_q = bh_q / a.Hkv;
    const int hk_q = bh_q - b_q * a.Hkv;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = (w * MB + mb) * 32 + l32;
      const int t = qb_q * C::BQ + r / G;
      const int hq = hk_q * G + (r % G);
      const bool valid = blk && t < a.T;
      const uint16_t* qp =
          a.q + b_q * a.q_sb + static_cast<int64_t>(t) * a.q_st + static_cast<int64_t>(hq) * D + 8 * h2;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        qraw[mb][ks] = u32x4{0u, 0u, 0u, 0u};
        if (valid) qraw[mb][ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      }
#pragma unroll
      for (int ks = 0; ks < C::KS / 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) traw[mb][ks][e] = float2{1.f, 0.f};
      if (a.rope && valid) {
        const float2* rt =
            a.rope + ((a.rope_batched ? static_cast<int64_t>(b_q) * a.T : 0) + t) * (D / 2) + 8 * h2;
#pragma unroll
        for (int ks = 0; ks < C::KS / 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) traw[mb][ks][e] = rt[16 * ks + e];
      }
    }
    qraw_lx = blk ? lx_q : -1;
  };

  for (int lx = lx_first; lx < lx_end; lx += lx_step) {
  int bh, qb;
  block_of(lx, bh, qb);
  if (qb >= a.n_qblocks) continue;  // padding block (uniform over the workgroup)
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const int t0 = qb * C::BQ;
  const int piece = split ? lx - (lx / a.nsplit) * a.nsplit : 0;
  // Chunked prefill: query row t is key slot t + qoff of the tile image
  // (0 for a whole-sequence prefill).  Every key index below is a slot.
  int qoff = 0;
  bool zero_out = false;
  if (a.start) {
    const int st = a.start[b];
    zero_out = !chunk_start_ok(st, a.max_start);
    qoff = zero_out ? 0 : st - chunk_kbase(st, a.W);
  }

  int tq[MB];  // token of this lane's query column in each row block
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) tq[mb] = t0 + ((w * MB + mb) * 32 + l32) / G;

  // ---- key range: masked edge tiles and the unmasked middle ----
  // The last key visible to query slot qs: qs itself (causal), or with no
  // causal mask qs + W - 1 (every key if W = 0), up to the last key slot.
  const int kmax = a.T - 1 + qoff;
  auto key_hi = [&](int qs) {
    if (!a.noncausal) return qs;
    return a.W > 0 ? min(kmax, qs + a.W - 1) : kmax;
  };
  const int q0 = t0 + qoff;                           // slot of the block's first query
  const int tlast = min(t0 + C::BQ, a.T) - 1 + qoff;  // slot of its last real query
  const int klo = a.W > 0 ? max(0, q0 - a.W + 1) : 0;
  int tile_lo = klo / kKeyTile;
  int tile_hi = key_hi(tlast) / kKeyTile;
  // tiles fully visible to every token of the block: k0 + 63 <= key_hi(q0)
  // and k0 > tlast - W
  int mid_lo = tile_lo;
  if (a.W > 0) {
    const int first_full = tlast - a.W + 1;                 // need k0 >= first_full
    mid_lo = max(tile_lo, (max(first_full, 0) + kKeyTile - 1) / kKeyTile);
  }
  const int mid_hi = min((key_hi(q0) + 1) / kKeyTile, tile_hi + 1);
  const int m_lo = min(mid_lo, mid_hi);
  const int m_hi = max(mid_hi, m_lo);

  // Logit shift.  With unit-RMS keys every logit lies within +-qbound
  // (63.2 log2 units).  Cached history is taken as stored, so its key rows
  // may have a larger RMS: the block's bound grows with the largest of them
  // over the block's whole tile range (every key piece of a split block
  // finds the same value), and where it passes kLogitCap the logit
  // accumulators start at minus the excess.  Unit-RMS caches give exactly 0.
  float s_init = 0.f;
  if constexpr (HMODE != 0) {
    const float* tm = a.tile_ms + static_cast<int64_t>(bh) * a.n_tiles;
    float m = 1.0f;
    for (int i = tile_lo + lane; i <= tile_hi; i += kWave) m = fmaxf(m, tm[i]);
    m = wave_max(m);
    s_init = -fmaxf(0.f, a.qbound * sqrtf(m) - kLogitCap);
    // the same in every lane (and in every wave and key piece of the block):
    // a scalar, so skipping the block is a uniform branch before any barrier
    s_init = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_init)));
    if ((HMODE == 1) != (s_init == 0.f)) continue;  // the other launch of the pair computes this block
  }

  // partial sums of output row (t, hq) for this key piece
  const int n_seq = a.batch_heads / a.Hkv;
  auto part_row = [&](int t, int hq) -> int64_t {
    return ((static_cast<int64_t>(piece) * n_seq + b) * a.T + t) * (static_cast<int64_t>(a.Hkv) * G) + hq;
  };
  if (split) {
    // this piece of the tile range (the masks above stay those of the block)
    const int n = tile_hi - tile_lo + 1;
    const int lo = tile_lo + (piece * n) / a.nsplit;
    tile_hi = tile_lo + ((piece + 1) * n) / a.nsplit - 1;
    tile_lo = lo;
    if (tile_hi < tile_lo) {
      // an empty piece adds nothing: zero partials for the block's rows
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = (w * MB + mb) * 32 + l32;
        const int t = t0 + r / G;
        if (t >= a.T) continue;
        const int64_t pr = part_row(t, hk * G + (r % G));
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < D / 2; d += 4) *reinterpret_cast<f32x4*>(a.part_o + pr * D + h2 * (D / 2) + d) = z;
        if (h2 == 0) a.part_l[pr] = 0.f;
      }
      continue;  // uniform over the workgroup, before any barrier
    }
  }

  // per-lane visible range of each row block: key in [lo_t, lo_t + span]
  int lo_t[MB], span[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int qs = tq[mb] + qoff;
    lo_t[mb] = a.W > 0 ? max(0, qs - a.W + 1) : 0;
    span[mb] = key_hi(qs) - lo_t[mb];
  }

  const u32x4* tsrc = a.tiles + static_cast<int64_t>(bh) * a.n_tiles * TL::CHUNKS;

  f32x16 o[MB][C::DB];
  f32x4 lacc[MB];  // row sums, accumulated on the matrix cores (layout below)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    lacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mb][db][i] = 0.f;
  }

  // ---- tile staging: four LDS buffers; tiles i-1 (its V still feeds the
  // pipelined PV), i and i+1 resident while the copy of tile i+2 streams
  // straight from global memory into LDS (global_load_lds_dwordx4: no register
  // staging, no LDS store instructions).  Each wave instruction copies 64
  // consecutive 16-byte chunks, so the LDS image of a tile equals its
  // workspace image.  Wave w copies the tile's chunks [w R 64, (w + 1) R 64)
  // in R rounds of 1 KB. ----
  constexpr int RND = TL::CHUNKS / C::THREADS;
  static_assert(TL::CHUNKS % C::THREADS == 0, "a tile is whole rounds of every wave");
  const uint32_t dma_lane = static_cast<uint32_t>(lane) * 16;
  auto gload = [&](int tile, int buf) {
    const u32x4* src = tsrc + static_cast<int64_t>(tile) * TL::CHUNKS + w * (RND * 64);
    dma_wave_share<RND>(src, dma_lane, tile_buf(buf) + w * (RND * 64));
  };
  // The first three tiles of the range start streaming into LDS before the
  // query prologue, so their latency overlaps the query loads.
  gload(tile_lo, 0);
  if (tile_lo + 1 <= tile_hi) gload(tile_lo + 1, 1);
  if (tile_lo + 2 <= tile_hi) gload(tile_lo + 2, 2);

  // ---- queries: load (unless prefetched), weightless RMS norm, scale,
  // RoPE, fp16 operands ----
  if (qraw_lx != lx) load_q(lx, true);
  half8 qf[MB][C::KS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const bool valid = tq[mb] < a.T;
    float x[C::KS][8];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) unpack_16x8(qraw[mb][ks], x[ks], a.in_f16);
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
#pragma unroll
      for (int ks = 0; ks < C::KS / 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = traw[mb][ks][e];
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

  // after computing tile `tile`: publish tile+2 (its copy was issued one step
  // earlier), then start tile+3 into the buffer of tile-1, which no wave reads
  // any more.  The barrier waits only for this wave's own tile copies
  // (vmcnt): LDS fragment reads of the next half-tile, which target tiles
  // that stay resident, remain in flight across it.  The empty asm statements
  // keep the compiler from moving memory accesses across the barrier.

  auto advance = [&](int tile) {
    const int rel = tile - tile_lo;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    if (tile + 3 <= tile_hi) gload(tile + 3, static_cast<unsigned>(rel + 3) % NBUF);
  };

  // Row sums on the matrix cores instead of vector dot products (head width
  // 64 is bound by vector issue, two exponentials per matrix item): one
  // v_mfma_f32_16x16x32_bf16 per 16-key P fragment, with a constant A of
  // ones and zeros.  That MFMA reads lane l of the fragment as column l % 16,
  // keys 8 (l / 16) ..: A row i takes k-blocks 0 and 2 (i < 8) or 1 and 3
  // (i >= 8), so output rows 0-7 hold the sums of columns 0-15 and rows 8-15
  // those of columns 16-31, over all 16 keys.  The epilogue picks each lane's
  // column from the accumulator layout (lane l holds rows 4 (l / 16) ..).
  bf16x8 aones;
  {
    const bool on = ((lane >> 4) & 1) == ((lane & 15) >> 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) aones[e] = static_cast<bf16_t>(on ? 1.0f : 0.0f);
  }

  // Edge tiles (a wave-uniform flag) overwrite the logits of invisible keys
  // with -inf, in a branch taken only on those tiles.
  auto mask_logits = [&](f32x16* sl, bool masked, int k0) {
    if (masked) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int kbase = k0 + 4 * h2 - lo_t[mb];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 8 * (i >> 2) + (i & 3);
          sl[mb][i] = static_cast<unsigned>(kbase + off) <= static_cast<unsigned>(span[mb]) ? sl[mb][i] : -INFINITY;
        }
      }
    }
  };

  // A half-step works on 32 keys.  Its matrix-core items alternate
  //   K item i:  S_out += K(tile_q, half kb_q) fragment i  x  q_hat fragment i
  //   V item i:  O     += V^T(tile_v, half kb_v) fragment i  x  P_in
  //              (and, on the first head-dim block, the row sums of P_in)
  // (a dependent MFMA chain on one accumulator runs at half rate, so the QK
  // chain is interleaved with the independent PV accumulators); between them
  // the vector ALUs turn S_in into P_out = exp2(S_in) (logits are bounded by
  // 63.2 in log2 units, so no running maximum is needed).  sched_barrier(0)
  // walls keep this order.
  //
  // LDS fragments stream through a queue of QD registers that runs
  // continuously across half-steps and tiles: the fragment of item j is read
  // QD items before its MFMA, the last QD reads of a half-step fetch the first
  // items of the next one, so the read latency stays hidden behind QD matrix
  // items and the queue never drains.  Every fragment address is a
  // compile-time offset from a per-half-step base.
  constexpr int NK = C::KS;
  constexpr int NI = NK + 2 * C::DB;  // items per half-step (NK == 2 * DB)
  static_assert(NK == 2 * C::DB, "K and V items alternate one to one");
  constexpr int QD = D == 128 ? kFragQueueD128 : kFragQueueD64;
  static_assert(NI % QD == 0, "queue slots line up across half-steps");
  const int k_lane = TL::k(l32, h2) * 16;  // bytes: key row l32, chunk h2
  const int v_lane = TL::v(l32, h2) * 16;  // bytes: head-dim row l32, chunk h2
  struct Half {
    const char* k;
    const char* v;
  };
  auto half_at = [&](int tile_q, int kb_q, int tile_v, int kb_v) -> Half {
    Half hb;
    // key rows 32 kb_q on; V chunks (8 keys each) 4 kb_v on
    // tiles at or after tile_lo: an unsigned remainder is a mask (the signed
    // one cost a dozen scalar instructions per half-step)
    const unsigned bk = static_cast<unsigned>(tile_q - tile_lo) % NBUF;
    const unsigned bv = static_cast<unsigned>(tile_v - tile_lo) % NBUF;
    hb.k = reinterpret_cast<const char*>(tile_buf(bk)) + k_lane + TL::k(32 * kb_q, 0) * 16;
    hb.v = reinterpret_cast<const char*>(tile_buf(bv)) + v_lane + (TL::v(0, 4 * kb_v) - TL::v(0, 0)) * 16;
    return hb;
  };
  // The same from ring byte offsets (NBUF and the tile size are powers of
  // two, so an offset wraps by masking): the tile loop steps three offsets
  // instead of recomputing them from tile indices.
  constexpr unsigned TB = TL::CHUNKS * 16;
  constexpr unsigned RING = NBUF * TB - TB;
  static_assert((NBUF & (NBUF - 1)) == 0 && (TB & (TB - 1)) == 0, "ring offsets wrap by masking");
  auto half_off = [&](unsigned oq, int kb_q, unsigned ov, int kb_v) -> Half {
    Half hb;
    hb.k = reinterpret_cast<const char*>(smem) + oq + k_lane + TL::k(32 * kb_q, 0) * 16;
    hb.v = reinterpret_cast<const char*>(smem) + ov + v_lane + (TL::v(0, 4 * kb_v) - TL::v(0, 0)) * 16;
    return hb;
  };
  auto frag = [&](const Half& hb, int j) -> u32x4 {
    const int i = j >> 1;
    // K item i: head dims 16 i .. 16 i + 15 (chunks 2 i, 2 i + 1)
    if ((j & 1) == 0) return *reinterpret_cast<const u32x4*>(hb.k + TL::k(0, 2 * i) * 16);
    // V item (st, db): head-dim rows 32 db on, keys 16 st on (chunks 2 st, 2 st + 1)
    const int st = i / C::DB, db = i % C::DB;
    return *reinterpret_cast<const u32x4*>(hb.v + (TL::v(32 * db, 2 * st) - TL::v(0, 0)) * 16);
  };
  u32x4 fq[QD];
  auto prime = [&](const Half& hb) {
#pragma unroll
    for (int j = 0; j < QD; ++j) fq[j] = frag(hb, j);
  };
  // do_qk / do_pv (std::true_type or std::false_type) select the logit and
  // the P V products; the exponentials run only in a half-step that has
  // both (the pipeline's fill has no P yet, its drain no logits to turn).
  auto half_step = [&](const Half& cur, const Half& nxt, f32x16* s_out, bf16x8 (*p_in)[2], f32x16* s_in,
                       bf16x8 (*p_out)[2], auto do_qk, auto do_pv) {
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value, EXP = QK && PV;
    constexpr bool SHIFTED = HMODE == 2;
    constexpr int NE = 16;  // logits per lane per row block
    // Head width 128 has one exponential per matrix item and packs each
    // pair one item late; at 64 every item has two, and packing at once
    // measured faster.
    constexpr bool kLagPack = D == 128;
    static_assert(!kLagPack || NE == NI, "one exponential per matrix item");
    float pend0[MB], pend1[MB];
    int pend_e = -1;
    auto pack_pair = [&](int mb, int e, float y0, float y1) {
      bf16x2 pr;
      pr[0] = static_cast<bf16_t>(y0);
      pr[1] = static_cast<bf16_t>(y1);
      uint32_t pw = __builtin_bit_cast(uint32_t, pr);
      asm volatile("" : "+v"(pw));
      pr = __builtin_bit_cast(bf16x2, pw);
      p_out[mb][e >> 3][e & 7] = pr[0];
      p_out[mb][e >> 3][(e & 7) + 1] = pr[1];
    };
    if constexpr (EXP) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(s_in[mb]));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s_out[mb][e] = SHIFTED ? s_init : 0.f;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 f = fq[j % QD];
      const int i = j >> 1;
      if ((j & 1) == 0) {
        if constexpr (QK) {
          const half8 kf = __builtin_bit_cast(half8, f);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            s_out[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[mb][i], s_out[mb], 0, 0, 0);
        }
      } else if constexpr (PV) {
        const int st = i / C::DB, db = i % C::DB;
        const bf16x8 vf = __builtin_bit_cast(bf16x8, f);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          o[mb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p_in[mb][st], o[mb][db], 0, 0, 0);
        if (db == 0) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            lacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aones, p_in[mb][st], lacc[mb], 0, 0, 0);
        }
      }
      fq[j % QD] = j + QD < NI ? frag(cur, j + QD) : frag(nxt, j + QD - NI);
      // the previous item's exponentials, packed one matrix item after they
      // were issued, so the transcendental unit's latency does not hold up
      // this wave's next MFMA
      if (pend_e >= 0) {
        for (int mb = 0; mb < MB; ++mb) pack_pair(mb, pend_e, pend0[mb], pend1[mb]);
        pend_e = -1;
      }
      // this item's slice of the exponentials.  The empty asm statements pin
      // them to this slot: the one on the whole S_in at the top of the
      // half-step stops the edge-tile mask from being folded into exp2
      // (exp2(-inf) = 0) and the exponentials from being hoisted; the one on
      // each output stops machine sinking from moving them into the next
      // block, past the matrix-core work they hide under.
      if constexpr (EXP && kLagPack) {
        // head width 128: one exponential per matrix item (16 per 16
        // items), so no item carries more vector work than the other wave's
        // MFMA covers; each pair is packed on the item after its second
        // exponential
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          float x = __builtin_amdgcn_exp2f(s_in[mb][j]);
          asm volatile("" : "+v"(x));
          if (j & 1)
            pend1[mb] = x;
          else
            pend0[mb] = x;
        }
        if (j & 1) pend_e = j - 1;
      } else if constexpr (EXP) {
        // head width 64: two exponentials per item, packed at once
#pragma unroll
        for (int e = (j * NE / NI) & ~1; e < (((j + 1) * NE / NI) & ~1); e += 2) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const float x0 = __builtin_amdgcn_exp2f(s_in[mb][e]);
            const float x1 = __builtin_amdgcn_exp2f(s_in[mb][e + 1]);
            pack_pair(mb, e, x0, x1);
          }
        }
      }
    }
    if (pend_e >= 0) {
      for (int mb = 0; mb < MB; ++mb) pack_pair(mb, pend_e, pend0[mb], pend1[mb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Software pipeline over half-tiles (32 keys): half-step k computes the
  // logits of half k on the matrix cores, turns the logits of half k-1 into
  // probabilities on the vector ALUs, and accumulates P V of half k-2.  Per
  // tile the two half-steps swap the roles of the S and P registers, so no
  // copies are needed.  One loop body serves every tile (a single copy keeps
  // register pressure low): in the first tile the "previous" P is zero over
  // valid V data.  The fill before the loop computes only the first logits,
  // the drain after it only the last P V.
  f32x16 sc[MB], sn[MB];          // logits: current half, next half
  bf16x8 pc[MB][2], pp[MB][2];    // probabilities: current half, previous half
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) pp[mb][st][e] = static_cast<bf16_t>(0.0f);

  // tiles 0, 1 and 2 of the range are resident after this barrier (the
  // explicit wait covers their copies)
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  // A wave whose columns all lie past the last query row (the short block of
  // a drafter) only copies its share of each tile and meets the barriers.
  // Only the SKIP instance tests for it: in the others the branch would cost
  // the common path about 2 % (register allocation and scheduling).
  const bool idle = SKIP && t0 + (w * MB * 32) / G >= a.T;
  // fill: S(first tile, 0..31) only
  if (!idle) {
    const Half h0 = half_at(tile_lo, 0, tile_lo, 0);
    prime(h0);
    half_step(h0, half_at(tile_lo, 1, tile_lo, 1), sc, pp, sn, pc, std::true_type{}, std::false_type{});
  }
  unsigned ocur = 0;  // ring offset of tile t's buffer
  for (int t = tile_lo; t <= tile_hi; ++t) {
    if (idle) {
      advance(t);
      continue;
    }
    // edge tiles: t < m_lo or t >= m_hi (m_lo <= m_hi)
    const bool masked = static_cast<unsigned>(t - m_lo) >= static_cast<unsigned>(m_hi - m_lo);
    const int k0 = t * kKeyTile;
    // tiles t - 1 and t + 1, held at the range's ends
    const unsigned oprev = t > tile_lo ? (ocur - TB) & RING : ocur;
    const unsigned onext = t < tile_hi ? (ocur + TB) & RING : ocur;
    const Half ha = half_off(ocur, 1, oprev, 1);
    const Half hb = half_off(onext, 0, ocur, 0);
    const Half hn = half_off(onext, 1, ocur, 1);   // half A of the next tile (or the drain)
    mask_logits(sc, masked, k0);
    // S(t, 32..63) and O += P(t-1, 32..63) V  ||  P(t, 0..31)
    half_step(ha, hb, sn, pp, sc, pc, std::true_type{}, std::true_type{});
    mask_logits(sn, masked, k0 + 32);
    // S(t+1, 0..31) and O += P(t, 0..31) V  ||  P(t, 32..63)
    half_step(hb, hn, sc, pc, sn, pp, std::true_type{}, std::true_type{});
    advance(t);
    ocur = (ocur + TB) & RING;
  }
  constexpr int CPC = D / 8;                     // 8-value chunks per column
  constexpr int NCH = MB * 32 * CPC;             // chunks per wave
  static_assert(NCH % kWave == 0, "whole chunk rounds");
  // Gate rows of the chunks this lane stores in the epilogue, loaded before
  // the drain (whose P V has no use for the query operands and logits, so
  // their registers hold these) so that their latency overlaps the drain and
  // the staging.
  u32x4 gpre[NCH / kWave];
#pragma unroll
  for (int it = 0; it < NCH / kWave; ++it) {
    const int k = it * kWave + lane;
    const int cl = k / CPC, d0 = (k % CPC) * 8;
    const int r = w * MB * 32 + cl;
    const int t = t0 + r / G;
    gpre[it] = u32x4{0u, 0u, 0u, 0u};
    if (!split && t < a.T)
      gpre[it] = *reinterpret_cast<const u32x4*>(a.gate + b * a.g_sb + static_cast<int64_t>(t) * a.g_st +
                                                 static_cast<int64_t>(hk * G + (r % G)) * D + d0);
  }
  // drain: O += P(last, 32..63) V only
  if (!idle) {
    const Half hd = half_at(tile_hi, 1, tile_hi, 1);
    half_step(hd, hd, sn, pp, sc, pc, std::false_type{}, std::true_type{});
  }
  // (only head width 128 runs persistent grids; at 64 the prefetch would
  // only cost the zeroing of the registers)
  if constexpr (D == 128) load_q(lx + lx_step, persistent && lx + lx_step < lx_end);

  // ---- epilogue: 1/sum, per-head output norm, then through LDS to row-major
  // order for the sigmoid gate and coalesced bf16 stores.  In the MFMA layout
  // a lane holds 4 consecutive dims of one (token, head) column, so direct
  // stores would leave every 128-byte line written in 16-byte pieces by
  // different instructions; staged, each lane loads 8 consecutive gate values
  // and stores 8 consecutive outputs, and a wave covers whole lines. ----
  __syncthreads();                              // every wave is done with the tiles
  float* ost = reinterpret_cast<float*>(smem) + w * (MB * 32 * OROW);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // column l32 of this lane: lanes 0-15 and 48-63 hold their own, lanes
    // 32-47 the sums of columns 16-31 that lanes 16-31 need, lanes 0-15
    // those of columns 0-15 that lanes 32-47 need
    const int src = lane < 16 ? lane : lane < 32 ? lane + 16 : lane < 48 ? lane - 32 : lane;
    const float ltot = __shfl(lacc[mb][0], src, kWave);
    if (split) {
      // a key piece hands on its unnormalized sums
      const int r = (w * MB + mb) * 32 + l32;
      const int t = t0 + r / G;
      if (h2 == 0 && t < a.T) a.part_l[part_row(t, hk * G + (r % G))] = ltot;
    }
    const float inv = split ? 1.0f : __builtin_amdgcn_rcpf(ltot);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mb][db][i] *= inv;
    float rsn = 1.0f;
    if (a.out_norm && !split) {
      float ss = 0.f;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) ss += o[mb][db][i] * o[mb][db][i];
      ss += __shfl_xor(ss, 32, kWave);
      rsn = __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.out_eps);
    }
    float* col = ost + (mb * 32 + l32) * OROW;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[mb][db][4 * grp + e] * rsn;
        *reinterpret_cast<f32x4*>(col + 32 * db + 8 * grp + 4 * h2) = v;
      }
  }
  // LDS accesses of one wave execute in order; the fence keeps the compiler
  // from reordering the reads below above the writes
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int it = 0; it < NCH / kWave; ++it) {
    const int k = it * kWave + lane;
    const int cl = k / CPC;                      // wave-local column
    const int d0 = (k % CPC) * 8;
    const int r = w * MB * 32 + cl;              // block column
    const int t = t0 + r / G;
    if (t < a.T && split) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(ost + cl * OROW + d0);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(ost + cl * OROW + d0 + 4);
      float* po = a.part_o + part_row(t, hk * G + (r % G)) * D + d0;
      *reinterpret_cast<f32x4*>(po) = v0;
      *reinterpret_cast<f32x4*>(po + 4) = v1;
    } else if (t < a.T) {
      const int hq = hk * G + (r % G);
      const u32x4 gw = gpre[it];
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(ost + cl * OROW + d0);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(ost + cl * OROW + d0 + 4);
      float g[8];
      unpack_16x8(gw, g, a.in_f16);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g[e]));
        y[e] = zero_out ? 0.f : (e < 4 ? v0[e] : v1[e - 4]) * sg;
      }
      u32x4 ow;
#pragma unroll
      for (int e = 0; e < 4; ++e) ow[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
      *reinterpret_cast<u32x4*>(a.out + b * a.o_sb + static_cast<int64_t>(t) * a.o_st + static_cast<int64_t>(hq) * D +
                                d0) = ow;
    }
  }
  // the staging area is the tile buffers: every wave is done reading it
  // before the next block's tile copies land there
  __syncthreads();
  }  // query blocks of this workgroup
}

// Key-split finish: CPC = D/8 lanes per output row, 8 dims each.  Sums the
// pieces' partials in piece order, then the prefill epilogue's arithmetic:
// 1/sum, the per-head RMS norm over D, y = o * sigmoid(g), bf16.
template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillCombineArgs a) {
  constexpr int CPC = D / 8;
  constexpr int RPB = 256 / CPC;
  const int64_t R = static_cast<int64_t>(a.B) * a.T * a.Hq;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / CPC;
  if (row >= R) return;  // whole groups of CPC lanes
  const int d0 = (threadIdx.x % CPC) * 8;
  const int hq = static_cast<int>(row % a.Hq);
  const int64_t bt = row / a.Hq;
  const int t = static_cast<int>(bt % a.T);
  const int b = static_cast<int>(bt / a.T);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float* po = a.part_o + (static_cast<int64_t>(s) * R + row) * D + d0;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(po);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(po + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += x0[e];
      acc[e + 4] += x1[e];
    }
    l += a.part_l[static_cast<int64_t>(s) * R + row];
  }
  const float inv = __builtin_amdgcn_rcpf(l);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc[e] *= inv;
    ss += acc[e] * acc[e];
  }
#pragma unroll
  for (int m = 1; m < CPC; m <<= 1) ss += __shfl_xor(ss, m, kWave);
  const float rsn = a.out_norm ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.out_eps) : 1.0f;
  const bool zero_out = a.start && !chunk_start_ok(a.start[b], a.max_start);
  const u32x4 gw = *reinterpret_cast<const u32x4*>(a.gate + b * a.g_sb + static_cast<int64_t>(t) * a.g_st +
                                                   static_cast<int64_t>(hq) * D + d0);
  float g[8];
  unpack_bf16x8(gw, g);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g[e]));
    y[e] = zero_out ? 0.f : acc[e] * rsn * sg;
  }
  u32x4 ow;
#pragma unroll
  for (int e = 0; e < 4; ++e) ow[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
  *reinterpret_cast<u32x4*>(a.out + b * a.o_sb + static_cast<int64_t>(t) * a.o_st + static_cast<int64_t>(hq) * D + d0) =
      ow;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {
// Launch shape per head width: waves per workgroup and 32-row MFMA blocks per
// wave.  Head width 128: 8 waves x 32 rows (two waves per SIMD, so one wave's
// exponentials overlap the other's matrix-core work).  Head width 64: the
// same shape needs half the registers, so two workgroups share a CU.
template <int D>
struct LaunchShape {
  static constexpr int NW = 8;
  static constexpr int MB = 1;
};

// Resident workgroups of one kernel on the current device: CUs times the
// occupancy the kernel's registers and LDS allow, cached per device in the
// caller's array (one per kernel instance).
constexpr int kMaxDev = 64;
template <typename K>
int resident_workgroups(K kernel, int threads, int* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  if (cache[dev] > 0) return cache[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  cache[dev] = cus * per_cu;
  return cache[dev];
}

template <int D, int G, bool SKIP, int HMODE>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  constexpr int NW = LaunchShape<D>::NW, MB = LaunchShape<D>::MB;
  using C = PrefillCfg<D, G, NW, MB>;
  auto kernel = prefill_kernel<D, G, NW, MB, SKIP, HMODE>;
  const int nlog = a.n_qblocks_pad * a.batch_heads;  // a multiple of 8
  int grid = nlog;
  if (a.nsplit > 1) {
    grid = a.n_qblocks * a.batch_heads * a.nsplit;
  } else if (D == 128 && a.W > 0) {
    // local layers run a persistent grid of at most one wave of resident
    // workgroups, a multiple of 8 so every XCD gets the same number
    static int resident[kMaxDev] = {};
    const int cap = resident_workgroups(kernel, C::THREADS, resident) & ~7;
    if (cap >= 8 && cap < nlog) grid = cap;
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

template <int D, int G, bool SKIP>
hipError_t launch_skip(const PrefillArgs& a, hipStream_t st) {
  if (!a.tile_ms) return launch_one<D, G, SKIP, 0>(a, st);
  // cached history: the blocks that need no logit shift, then those that do
  hipError_t e = launch_one<D, G, SKIP, 1>(a, st);
  if (e != hipSuccess) return e;
  return launch_one<D, G, SKIP, 2>(a, st);
}

template <int D, int G>
hipError_t launch_dg(const PrefillArgs& a, hipStream_t st) {
  constexpr int NW = LaunchShape<D>::NW, MB = LaunchShape<D>::MB;
  using C = PrefillCfg<D, G, NW, MB>;
  // a sequence shorter than one query block leaves whole waves without rows
  return a.T < C::BQ ? launch_skip<D, G, true>(a, st) : launch_skip<D, G, false>(a, st);
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

int prefill_rows_per_block(int d, int) {
  return d == 128 ? LaunchShape<128>::NW * LaunchShape<128>::MB * 32 : LaunchShape<64>::NW * LaunchShape<64>::MB * 32;
}

int prefill_qblock_group() { return kQBlockGroup; }

int prefill_key_split(int64_t n_blocks, int64_t max_tiles, int cus) {
  const int64_t kFillBlocks = cus, kTargetWorkgroups = cus, kMaxPieces = 16;
  if (n_blocks <= 0 || n_blocks >= kFillBlocks) return 1;
  int64_t s = (kTargetWorkgroups + n_blocks - 1) / n_blocks;
  s = std::min(s, std::min(kMaxPieces, max_tiles / 2));
  return static_cast<int>(std::max<int64_t>(s, 1));
}

hipError_t launch_prefill_combine(int d, const PrefillCombineArgs& a, hipStream_t st) {
  const int64_t R = static_cast<int64_t>(a.B) * a.T * a.Hq;
  if (R == 0) return hipSuccess;
  const int rpb = 256 / (d / 8);
  const unsigned blocks = static_cast<unsigned>((R + rpb - 1) / rpb);
  if (d == 64)
    hipLaunchKernelGGL(prefill_combine_kernel<64>, dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_combine_kernel<128>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill(int d, int g, const PrefillArgs& a, hipStream_t st) {
  return d == 64 ? launch_d<64>(g, a, st) : launch_d<128>(g, a, st);
}

}  // namespace muse
