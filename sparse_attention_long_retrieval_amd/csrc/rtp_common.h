// Device helpers shared by the gfx950 kernels of the head-wise sparse attention step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define RTP_D 128
#define RTP_R 16
#define RTP_MAX_KV 64

namespace rtp {

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16, round to nearest even of the exact fp64 value (no double rounding
// through fp32).  Values inside the normal fp32 range; smaller magnitudes go
// through fp32 (they never occur for the caches and index this library writes).
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint32_t sign = (uint32_t)(u >> 63);
  int e = (int)((u >> 52) & 0x7ff);
  if (e == 0 || e - 1023 < -126) return f32_to_bf16((float)x);
  uint64_t mant = u & ((1ull << 52) - 1);
  // bf16 payload without sign: exponent (8 bits) | top 7 mantissa bits
  uint32_t body = ((uint32_t)(e - 1023 + 127) << 7) | (uint32_t)(mant >> 45);
  uint64_t rem = mant & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rem > half || (rem == half && (body & 1u))) body += 1;  // carry may bump the exponent
  return (uint16_t)((sign << 15) | (body & 0x7fffu));
}

// ------------------------------------------------------------------ ordering

// Monotone map of fp32 to uint32: a < b  <=>  ord(a) < ord(b) (no NaN).
__device__ __forceinline__ uint32_t f32_ord(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------ wave64 reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Key of the absolute score grid with bins of width 1/inv_delta.
__device__ __forceinline__ int score_key(float s, float inv_delta) {
  float k = floorf(s * inv_delta);
  k = fminf(fmaxf(k, -1.0e9f), 1.0e9f);
  return (int)k;
}

}  // namespace rtp
