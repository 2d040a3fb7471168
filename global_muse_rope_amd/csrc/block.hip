// The attention half of a decoder block around the layer (Muse Spark Open
// deep dive, section 2.1 forward walk; section 5.1 for Glimmer, 5.2-5.3 for
// Spark): input RMSNorm, the q/k/v/gate projections, the layer, o_proj, the
// post-attention norm and the residual.
//
// The two projections are plain GEMMs and go to hipBLASLt; the norms and the
// residual are row kernels here, one workgroup per token row:
//   input_layernorm: centered RMSNorm, x / sqrt(mean(x^2) + 1e-5) * (1 + w),
//     the gain formed and applied in fp32, h kept as a pair of bf16 rows
//     (h_hi = bf16(h), h_lo = bf16(h - h_hi)) so the projection GEMM (bf16
//     operands, fp32 out) sees h to about 16 bits;
//   the projections' fp32 sum of the two halves is handed to the layer with
//     q, k and the gate in fp16 (v in bf16, the type of the layer's value
//     product), and o_proj's output stays fp32 into the residual;
//   Glimmer: out = x + a / sqrt(mean(a^2) + 1e-8) * (1 + w_post);
//   Spark:   out = alpha * x + beta * a / sqrt(mean(a^2) + 1e-8), with
//     beta = sigmoid(g / T), alpha = sqrt(max(sigmoid(-g / T) (1 + beta), 1e-3))
//     (the norm-preserving residual gate, its per-channel coefficients in
//     fp32, computed once per call).
#include <hipblaslt/hipblaslt.h>

#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "kernels.h"

namespace muse {

namespace {
constexpr int kRowThreads = 256;
constexpr int kMaxChunksPerThread = kBlockMaxHidden / 8 / kRowThreads;

// sum over the workgroup (4 waves)
__device__ __forceinline__ float row_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

__device__ __forceinline__ float sigmoidf_(float x) {
  return 1.0f / (1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
}  // namespace

__global__ __launch_bounds__(kRowThreads) void block_input_norm_kernel(BlockNormArgs a) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nch = a.hidden / 8;
  const uint16_t* xr = a.x + row * a.hidden;
  float v[kMaxChunksPerThread][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    u32x4 w = {0, 0, 0, 0};
    if (c < nch) w = *reinterpret_cast<const u32x4*>(xr + 8 * c);
    unpack_bf16x8(w, v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
  }
  ss = row_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / a.hidden + a.eps);
  uint16_t* orow = a.out + row * a.hidden;
  uint16_t* lrow = a.out_lo + row * a.hidden;
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    if (c >= nch) continue;
    float g[8];
    unpack_bf16x8(*reinterpret_cast<const u32x4*>(a.w + 8 * c), g);
    u32x4 o, ol;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float h0 = v[i][2 * e] * rs * (1.0f + g[2 * e]), h1 = v[i][2 * e + 1] * rs * (1.0f + g[2 * e + 1]);
      o[e] = pack_bf16x2(h0, h1);
      ol[e] = pack_bf16x2(h0 - __uint_as_float(o[e] << 16), h1 - __uint_as_float(o[e] & 0xffff0000u));
    }
    *reinterpret_cast<u32x4*>(orow + 8 * c) = o;
    *reinterpret_cast<u32x4*>(lrow + 8 * c) = ol;
  }
}

// One workgroup per token row: the projection of h as the sum of its hi and
// lo halves (fp32), q / k / gate written as fp16 and v as bf16.
__global__ __launch_bounds__(kRowThreads) void block_proj_prep_kernel(BlockProjPrepArgs a) {
  const int64_t row = blockIdx.x;
  const float* hi = a.proj + row * a.n;
  const float* lo = a.proj + (a.rows + row) * a.n;
  uint16_t* out = a.out + row * a.n;
  for (int c = threadIdx.x * 8; c < a.n; c += kRowThreads * 8) {
    const f32x4 h0 = *reinterpret_cast<const f32x4*>(hi + c), h1 = *reinterpret_cast<const f32x4*>(hi + c + 4);
    const f32x4 l0 = *reinterpret_cast<const f32x4*>(lo + c), l1 = *reinterpret_cast<const f32x4*>(lo + c + 4);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = h0[e] + l0[e];
      x[e + 4] = h1[e] + l1[e];
    }
    // column ranges are multiples of 8: a chunk lies in one of them
    const bool v_cols = c >= a.k_end && c < a.v_end;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = v_cols ? pack_bf16x2(x[2 * e], x[2 * e + 1]) : pack_f16x2(x[2 * e], x[2 * e + 1]);
    *reinterpret_cast<u32x4*>(out + c) = w;
  }
}

__global__ __launch_bounds__(kRowThreads) void block_residual_kernel(BlockResidualArgs a) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nch = a.hidden / 8;
  const float* ar = a.branch + row * a.hidden;
  const uint16_t* xr = a.x + row * a.hidden;
  float v[kMaxChunksPerThread][8];
  u32x4 xw[kMaxChunksPerThread];  // the residual stream, fetched while the branch's norm is reduced
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = w0;
    xw[i] = u32x4{0, 0, 0, 0};
    if (c < nch) {
      w0 = *reinterpret_cast<const f32x4*>(ar + 8 * c);
      w1 = *reinterpret_cast<const f32x4*>(ar + 8 * c + 4);
      xw[i] = *reinterpret_cast<const u32x4*>(xr + 8 * c);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[i][e] = w0[e];
      v[i][e + 4] = w1[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
  }
  ss = row_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / a.hidden + a.eps);
  uint16_t* orow = a.out + row * a.hidden;
#pragma unroll
  for (int i = 0; i < kMaxChunksPerThread; ++i) {
    const int c = threadIdx.x + i * kRowThreads;
    if (c >= nch) continue;
    float x[8], y[8];
    unpack_bf16x8(xw[i], x);
    if (a.coef) {
      // Spark: norm-preserving residual gate over the weightless-normed branch
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const f32x4 ab = *reinterpret_cast<const f32x4*>(a.coef + 2 * (8 * c + e));  // (alpha, beta) x 2
        y[e] = ab[0] * x[e] + ab[1] * (v[i][e] * rs);
        y[e + 1] = ab[2] * x[e + 1] + ab[3] * (v[i][e + 1] * rs);
      }
    } else {
      // Glimmer: centered post-norm, then the plain residual add
      float g[8];
      unpack_bf16x8(*reinterpret_cast<const u32x4*>(a.post_norm + 8 * c), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[e] + v[i][e] * rs * (1.0f + g[e]);
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
    *reinterpret_cast<u32x4*>(orow + 8 * c) = o;
  }
}

// The residual gate's coefficients depend on the channel only: one pass
// per call turns the parameter g into (alpha, beta) pairs for every row.
__global__ __launch_bounds__(kRowThreads) void block_gate_coef_kernel(const float* gate, float2* coef, int hidden,
                                                                      float temperature, float alpha_sq_floor) {
  const int i = blockIdx.x * kRowThreads + threadIdx.x;
  if (i >= hidden) return;
  const float w = gate[i] / temperature;
  const float beta = sigmoidf_(w);
  const float alpha = sqrtf(fmaxf(sigmoidf_(-w) * (1.0f + beta), alpha_sq_floor));
  coef[i] = make_float2(alpha, beta);
}

hipError_t launch_block_gate_coef(const float* gate, float2* coef, int hidden, float temperature,
                                  float alpha_sq_floor, hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>((hidden + kRowThreads - 1) / kRowThreads);
  hipLaunchKernelGGL(block_gate_coef_kernel, dim3(blocks), dim3(kRowThreads), 0, st, gate, coef, hidden, temperature,
                     alpha_sq_floor);
  return hipGetLastError();
}

hipError_t launch_block_input_norm(const BlockNormArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(block_input_norm_kernel, dim3(static_cast<unsigned>(a.rows)), dim3(kRowThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_block_proj_prep(const BlockProjPrepArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(block_proj_prep_kernel, dim3(static_cast<unsigned>(a.rows)), dim3(kRowThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_block_residual(const BlockResidualArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(block_residual_kernel, dim3(static_cast<unsigned>(a.rows)), dim3(kRowThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMM through hipBLASLt: out[rows, n] = act[rows, k] * w[n, k]^T, all
// row-major, bf16 operands, fp32 accumulation and fp32 out.  In hipBLASLt's column-major terms
// that is D[n, rows] = op_T(W') * act', with W' = w viewed as [k, n] and
// act' = act viewed as [k, rows].  One handle per device, created on first
// use, and a record of the algorithm chosen per (device, shape): host state
// only; the caller's workspace is the GEMM's scratch.  An ordinary call
// never waits for the device: it runs the recorded algorithm, or on the
// first call of a shape the heuristic's first choice (and records it).  A
// tuning call (`tune`) times the heuristic's top candidates on its own
// operands instead (a few runs each, then a wait for the stream) and
// records the fastest for the calls that follow.
// ---------------------------------------------------------------------------
namespace {
std::mutex g_lt_mu;
hipblasLtHandle_t g_lt[64] = {};
constexpr int kTuneCandidates = 16;
using GemmKey = std::tuple<int, int64_t, int64_t, int64_t, size_t>;
std::map<GemmKey, hipblasLtMatmulAlgo_t> g_algo;

// Fastest of the candidates on stream st (one warm-up run, then two timed
// runs each); -1 if none runs.
int fastest_candidate(hipblasLtHandle_t h, hipblasLtMatmulDesc_t desc, hipblasLtMatrixLayout_t la,
                      hipblasLtMatrixLayout_t lb, hipblasLtMatrixLayout_t lc, const void* act, const void* w,
                      void* out, void* ws, size_t wsb, hipStream_t st, const hipblasLtMatmulHeuristicResult_t* res,
                      int found) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return found > 0 ? 0 : -1;
  }
  const float one = 1.0f, zero = 0.0f;
  int best = -1;
  float best_ms = 0.f;
  for (int i = 0; i < found; ++i) {
    auto run = [&]() {
      return hipblasLtMatmul(h, desc, &one, w, la, act, lb, &zero, out, lc, out, lc, &res[i].algo, ws, wsb, st) ==
             HIPBLAS_STATUS_SUCCESS;
    };
    if (!run()) continue;
    if (hipEventRecord(e0, st) != hipSuccess || !run() || !run() || hipEventRecord(e1, st) != hipSuccess ||
        hipEventSynchronize(e1) != hipSuccess)
      continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) continue;
    if (best < 0 || ms < best_ms) {
      best = i;
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return best;
}
}  // namespace

int block_gemm(int64_t rows, int64_t n, int64_t k, const void* act, const void* w, float* out, void* ws,
               size_t ws_bytes, hipStream_t st, char* err, size_t errlen, bool tune) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    snprintf(err, errlen, "no current device");
    return 1;
  }
  hipblasLtHandle_t h;
  {
    std::lock_guard<std::mutex> lk(g_lt_mu);
    if (!g_lt[dev] && hipblasLtCreate(&g_lt[dev]) != HIPBLAS_STATUS_SUCCESS) {
      g_lt[dev] = nullptr;
      snprintf(err, errlen, "hipblasLtCreate failed");
      return 1;
    }
    h = g_lt[dev];
  }
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  int rc = 1;
  do {
    if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) break;
    const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) != HIPBLAS_STATUS_SUCCESS)
      break;
    if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, k, n, k) != HIPBLAS_STATUS_SUCCESS) break;
    if (hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, k, rows, k) != HIPBLAS_STATUS_SUCCESS) break;
    if (hipblasLtMatrixLayoutCreate(&lc, HIP_R_32F, n, rows, n) != HIPBLAS_STATUS_SUCCESS) break;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) break;
    const uint64_t wsb = ws_bytes;
    if (hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb)) !=
        HIPBLAS_STATUS_SUCCESS)
      break;
    const GemmKey key{dev, rows, n, k, ws_bytes};
    hipblasLtMatmulAlgo_t algo;
    bool have = false;
    {
      std::lock_guard<std::mutex> lk(g_lt_mu);
      const auto it = g_algo.find(key);
      if (it != g_algo.end()) {
        algo = it->second;
        have = true;
      }
    }
    if (!have || tune) {
      hipblasLtMatmulHeuristicResult_t res[kTuneCandidates];
      int found = 0;
      if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, lc, lc, pref, tune ? kTuneCandidates : 1, res, &found) !=
              HIPBLAS_STATUS_SUCCESS ||
          found < 1) {
        snprintf(err, errlen, "hipBLASLt found no algorithm for %lld x %lld x %lld", static_cast<long long>(rows),
                 static_cast<long long>(n), static_cast<long long>(k));
        rc = 2;
        break;
      }
      int pick = 0;
      if (tune && found > 1) {
        pick = fastest_candidate(h, desc, la, lb, lc, act, w, out, ws, wsb, st, res, found);
        if (pick < 0) pick = 0;
      }
      std::lock_guard<std::mutex> lk(g_lt_mu);
      g_algo[key] = res[pick].algo;
      algo = res[pick].algo;
    }
    const float one = 1.0f, zero = 0.0f;
    if (hipblasLtMatmul(h, desc, &one, w, la, act, lb, &zero, out, lc, out, lc, &algo, ws, wsb, st) !=
        HIPBLAS_STATUS_SUCCESS) {
      snprintf(err, errlen, "hipblasLtMatmul failed");
      rc = 2;
      break;
    }
    rc = 0;
  } while (false);
  if (rc == 1) snprintf(err, errlen, "hipBLASLt descriptor setup failed");
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (lc) hipblasLtMatrixLayoutDestroy(lc);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return rc;
}

}  // namespace muse
