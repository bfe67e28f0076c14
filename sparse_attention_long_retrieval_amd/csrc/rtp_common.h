// Device helpers shared by the gfx950 kernels of the head-wise sparse attention step.
#pragma once

#include <climits>

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

// sin and cos of the RoPE angle pos * theta (theta from the fp64 frequency table): the
// angle is reduced to [0, 1) revolutions in fp64, then the hardware sin / cos take it
// in revolutions.  Used for queries only (outputs carry a tolerance); cached keys are
// rotated with fp64 sincos.
__device__ __forceinline__ void rope_sincos(int pos, double theta, float& sn, float& cs) {
  const double rev = (double)pos * theta * 0.15915494309189535;
  const float f = (float)(rev - floor(rev));
  sn = __builtin_amdgcn_sinf(f);
  cs = __builtin_amdgcn_cosf(f);
}

// Rotate the pair (x, y) by the angle with cosine c and sine s, then scale.  Each
// operation rounds on its own (no contraction into fma), so every kernel that
// rotates a query gets the same bits.
__device__ __forceinline__ void rope_rotate(float x, float y, float c, float s, float scale,
                                            float& r0, float& r1) {
#pragma clang fp contract(off)
  r0 = (x * c - y * s) * scale;
  r1 = (y * c + x * s) * scale;
}

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

// ------------------------------------------------------------------ wave64 scans

// Inclusive scans over the 64 lanes of a wave on DPP: row shifts by 1, 2, 4, 8
// within each row of 16 lanes, then the broadcasts of lane 15 into rows 1 and 3
// and of lane 31 into rows 2 and 3 (GFX9 DPP controls).  Every step is a VALU
// move, no LDS round trip.  A lane whose source is outside its row (or whose row
// is masked off) takes the identity.  Reductions read lane 63.
namespace dpp {
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t mov(uint32_t ident, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, CTRL, ROWS, 0xf, false);
}
}  // namespace dpp

// x of the lane that supplies step CTRL, or ident; 32-bit payloads.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x, uint32_t ident, Op op) {
  x = op(x, dpp::mov<dpp::kShr1, 0xf>(ident, x));
  x = op(x, dpp::mov<dpp::kShr2, 0xf>(ident, x));
  x = op(x, dpp::mov<dpp::kShr4, 0xf>(ident, x));
  x = op(x, dpp::mov<dpp::kShr8, 0xf>(ident, x));
  x = op(x, dpp::mov<dpp::kBcast15, 0xa>(ident, x));
  x = op(x, dpp::mov<dpp::kBcast31, 0xc>(ident, x));
  return x;
}
// 64-bit payloads: both halves move with the same control.
template <class Op>
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long x,
                                                            unsigned long long ident, Op op) {
  auto step = [&](auto mv) {
    const uint32_t lo = mv((uint32_t)ident, (uint32_t)x);
    const uint32_t hi = mv((uint32_t)(ident >> 32), (uint32_t)(x >> 32));
    x = op(x, ((unsigned long long)hi << 32) | lo);
  };
  step([](uint32_t i, uint32_t v) { return dpp::mov<dpp::kShr1, 0xf>(i, v); });
  step([](uint32_t i, uint32_t v) { return dpp::mov<dpp::kShr2, 0xf>(i, v); });
  step([](uint32_t i, uint32_t v) { return dpp::mov<dpp::kShr4, 0xf>(i, v); });
  step([](uint32_t i, uint32_t v) { return dpp::mov<dpp::kShr8, 0xf>(i, v); });
  step([](uint32_t i, uint32_t v) { return dpp::mov<dpp::kBcast15, 0xa>(i, v); });
  step([](uint32_t i, uint32_t v) { return dpp::mov<dpp::kBcast31, 0xc>(i, v); });
  return x;
}
__device__ __forceinline__ uint32_t lane63_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ unsigned long long lane63_u64(unsigned long long x) {
  return ((unsigned long long)lane63_u32((uint32_t)(x >> 32)) << 32) | lane63_u32((uint32_t)x);
}

__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t x) {
  return wave_scan_u32(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ unsigned long long wave_incl_sum_u64(unsigned long long x) {
  return wave_scan_u64(x, 0ull, [](unsigned long long a, unsigned long long b) { return a + b; });
}

// ------------------------------------------------------------------ wave64 reductions

__device__ __forceinline__ float wave_max(float v) {
  const uint32_t r = wave_scan_u32(__float_as_uint(v), __float_as_uint(-INFINITY),
                                   [](uint32_t a, uint32_t b) {
                                     return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
                                   });
  return __uint_as_float(lane63_u32(r));
}
__device__ __forceinline__ float wave_sum(float v) {
  const uint32_t r = wave_scan_u32(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float(lane63_u32(r));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  const unsigned long long r =
      wave_scan_u64((unsigned long long)__double_as_longlong(v), 0ull,
                    [](unsigned long long a, unsigned long long b) {
                      return (unsigned long long)__double_as_longlong(
                          __longlong_as_double((long long)a) + __longlong_as_double((long long)b));
                    });
  return __longlong_as_double((long long)lane63_u64(r));
}
__device__ __forceinline__ int wave_max_i(int v) {
  const uint32_t r = wave_scan_u32((uint32_t)v, (uint32_t)INT_MIN, [](uint32_t a, uint32_t b) {
    return (uint32_t)max((int)a, (int)b);
  });
  return (int)lane63_u32(r);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return lane63_u32(wave_scan_u32(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return lane63_u32(wave_scan_u32(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }));
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  return lane63_u64(wave_incl_sum_u64(v));
}

// Key of the absolute score grid with bins of width 1/inv_delta (clamped to
// +-1e9 so that differences of keys stay inside int; -inf maps to -1e9).
__device__ __forceinline__ int score_key(float s, float inv_delta) {
  return (int)__builtin_amdgcn_fmed3f(floorf(s * inv_delta), -1.0e9f, 1.0e9f);
}

}  // namespace rtp
