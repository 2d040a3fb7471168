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
  const int pos = a.positions ? a.positions[row] : static_cast<int>(row % a.T);
  float s, c;
  rope_sincos(pos, j, D, a.log2_theta, &s, &c);
  a.table[gt] = make_float2(c, s);
}

// ---------------------------------------------------------------------------
// Prefill key/value preparation: one 64-key tile of one (sequence, KV head)
// per workgroup.  Writes the tile image the attention kernel copies straight
// into LDS: k_hat as fp16 key rows and V transposed to head-dim rows (bf16),
// both with one pad chunk per row (layout in TileLayout).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void kv_prep_kernel(KvPrepArgs a) {
  constexpr int BK = kKeyTile;
  constexpr int RUN = D / 8;  // elements per thread in each half of the head
  __shared__ uint16_t vs[BK][D + 8];
  // KV heads vary fastest over the grid: the workgroups of one tile's heads
  // run together and read each token's row of all heads in one pass
  const int tile = blockIdx.x / a.Hkv;
  const int hk = blockIdx.x - tile * a.Hkv;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int r = tid >> 2;          // key within the tile
  const int qq = tid & 3;          // quarter of each half of the head
  const int tok = tile * BK + r;
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;

  // All loads of the tile (raw keys, values and RoPE rows) are issued
  // before the first use so their latencies overlap.  Rows past the end of
  // the sequence repeat the last row: they are never visible to a query (the
  // attention kernel masks them before the exponential), and finite values
  // keep p = 0 from meeting a non-finite V.
  const int tl = min(tok, a.T - 1);
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
  using TL = TileLayout<D>;
  u32x4* tdst = a.tiles + (bh * a.n_tiles + tile) * TL::CHUNKS;
  u32x4* kdst = tdst + r * TL::KROW;
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
    kdst[c0] = w0;
    kdst[c1] = w1;
  }
  // the pad chunks are written too (zeros), so every line of the tile image
  // is written whole
  if (qq == 0) kdst[D / 8] = u32x4{0, 0, 0, 0};

  __syncthreads();
  u32x4* vdst = tdst + TL::KCHUNKS;
  constexpr int CHUNKS = D * BK / 8;  // 16-byte chunks of the transposed tile
  for (int ci = tid; ci < CHUNKS; ci += 256) {
    const int d = ci / (BK / 8);
    const int pc = ci % (BK / 8);  // logical chunk: 16-key group g16 = pc/2, half hh = pc%2
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
    vdst[d * TL::VROW + pc] = w;
    if (pc == 0) vdst[d * TL::VROW + BK / 8] = u32x4{0, 0, 0, 0};
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
  if (d == 64) hipLaunchKernelGGL((kv_prep_kernel<64>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((kv_prep_kernel<128>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace muse
