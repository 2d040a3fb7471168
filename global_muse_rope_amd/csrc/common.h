// Shared device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muse {

typedef _Float16 half_t;
typedef __bf16 bf16_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  bf16_t h = static_cast<bf16_t>(x);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<bf16_t>(lo);
  v[1] = static_cast<bf16_t>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v;
  v[0] = static_cast<half_t>(lo);
  v[1] = static_cast<half_t>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 held in a 16-byte word into floats.
__device__ __forceinline__ void unpack_bf16x8(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Unpack 8 fp16 held in a 16-byte word into floats.
__device__ __forceinline__ void unpack_f16x8(const u32x4& w, float* f) {
  const half8 h = __builtin_bit_cast(half8, w);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(h[i]);
}

// 8 values of a 16-bit input tensor: fp16 if f16, else bf16.
__device__ __forceinline__ void unpack_16x8(const u32x4& w, float* f, bool f16) {
  if (f16)
    unpack_f16x8(w, f);
  else
    unpack_bf16x8(w, f);
}

__device__ __forceinline__ float bits16_to_f32(uint16_t b, bool f16) {
  return f16 ? static_cast<float>(__builtin_bit_cast(half_t, b)) : bf16_bits_to_f32(b);
}

// OCP E4M3 code of x (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals, no infinities; 0x7F is NaN): round to nearest, ties to an even
// mantissa, finite magnitudes beyond 448 saturate to 448, NaN gives 0x7F.
__device__ __forceinline__ uint8_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax != ax) return 0x7F;
  if (ax >= 448.0f) return static_cast<uint8_t>(sign | 0x7Eu);
  if (ax < 0.015625f) {                     // below 2^-6: multiples of 2^-9
    const int m = static_cast<int>(rintf(ax * 512.0f));  // exact scaling, ties to even; 8 = 2^-6
    return static_cast<uint8_t>(sign | static_cast<uint32_t>(m));
  }
  int e = static_cast<int>((u >> 23) & 0xFFu) - 127;  // -6 .. 8
  uint32_t keep = (u >> 20) & 0x7u;
  const uint32_t rem = u & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0u;
    ++e;
  }
  return static_cast<uint8_t>(sign | (static_cast<uint32_t>(e + 7) << 3) | keep);
}

// Eight E4M3 codes (one per byte, lowest first) to bf16, exactly (every
// E4M3 value has a bf16 representation).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 w) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true));
  return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// RoPE angle pos * theta^(-2j/D), formed and reduced to [-pi, pi] in fp64
// (positions reach 2^20, where an fp32 angle would carry errors of 0.06 rad),
// then sine and cosine in fp32.  log2_theta = log2(theta).
__device__ __forceinline__ void rope_sincos(int pos, int j, int d, double log2_theta,
                                            float* s, float* c) {
  const double inv_freq = exp2(-(2.0 * j / d) * log2_theta);
  const double a = static_cast<double>(pos) * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  const double r = a - two_pi * rint(a * (1.0 / two_pi));
  sincosf(static_cast<float>(r), s, c);
}

}  // namespace muse
