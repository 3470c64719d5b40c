// Device-side microscaling formats for gfx950.
//
// Element formats E2M1 / E2M3 / E4M3 and the E4M3 block scale of MicroQonv's
// NVFP4-style quantizer (arXiv 2609.28358, §II-D and §III-A).  Rounding works
// on the fp32 bit pattern: subnormal values by an exact power-of-two rescale
// and a round-to-integer, normal values by rounding the 23-bit mantissa to the
// format's width with carry into the exponent.  Both are the IEEE
// round-to-nearest-even of the value onto the format grid; values at or above
// the format maximum saturate to it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum { FMT_E2M1 = 1, FMT_E2M3 = 2, FMT_E4M3 = 3 };

template <int FMT> struct Fmt;
template <> struct Fmt<FMT_E2M1> {
  static constexpr int MB = 1, BIAS = 1, SIGN = 3, BITS = 4, MAXCODE = 7;
  static constexpr float MAXV = 6.0f;
};
template <> struct Fmt<FMT_E2M3> {
  static constexpr int MB = 3, BIAS = 1, SIGN = 5, BITS = 6, MAXCODE = 31;
  static constexpr float MAXV = 7.5f;
};
template <> struct Fmt<FMT_E4M3> {
  static constexpr int MB = 3, BIAS = 7, SIGN = 7, BITS = 8, MAXCODE = 126;
  static constexpr float MAXV = 448.0f;
};
using ScaleFmt = Fmt<FMT_E4M3>;

// Bytes of one 8x8 block of codes.
template <int FMT> constexpr int block_bytes() { return Fmt<FMT>::BITS * 8; }

// 2^k as a float for small k (compile time).
__host__ __device__ constexpr float pow2(int k) {
  return k >= 0 ? float(1ull << k) : 1.0f / float(1ull << -k);
}

// Round-to-nearest-even magnitude code of v >= 0 (v may be +inf).
template <class F>
__device__ __forceinline__ uint32_t rne_code(float v) {
  if (!(v < F::MAXV)) return F::MAXCODE;
  constexpr float MIN_NORMAL = pow2(1 - F::BIAS);
  if (v < MIN_NORMAL) {
    // subnormal grid step 2^(1-BIAS-MB): code = nearest integer of v / step
    return static_cast<uint32_t>(__builtin_rintf(v * pow2(F::MB + F::BIAS - 1)));
  }
  constexpr int SH = 23 - F::MB;
  uint32_t b = __float_as_uint(v);
  b += ((1u << (SH - 1)) - 1u) + ((b >> SH) & 1u);
  return (b >> SH) - static_cast<uint32_t>((127 - F::BIAS) << F::MB);
}

// Stochastic rounding: with lo <= v < hi the neighbouring grid points, round
// up iff u * (hi - lo) < v - lo (both fp32 operations exact).
template <class F>
__device__ __forceinline__ uint32_t sr_code(float v, float u) {
  if (!(v < F::MAXV)) return F::MAXCODE;
  constexpr float MIN_NORMAL = pow2(1 - F::BIAS);
  uint32_t lo;
  float lov, delta;
  if (v < MIN_NORMAL) {
    constexpr float STEP = pow2(1 - F::BIAS - F::MB);
    float q = __builtin_floorf(v * pow2(F::MB + F::BIAS - 1));
    lo = static_cast<uint32_t>(q);
    lov = q * STEP;
    delta = STEP;
  } else {
    constexpr int SH = 23 - F::MB;
    uint32_t b = __float_as_uint(v);
    uint32_t t = b & ~((1u << SH) - 1u);
    lov = __uint_as_float(t);
    lo = (t >> SH) - static_cast<uint32_t>((127 - F::BIAS) << F::MB);
    delta = __uint_as_float((b & 0x7F800000u) - (static_cast<uint32_t>(F::MB) << 23));
  }
  float diff = v - lov;
  float thr = u * delta;
  return lo + (thr < diff ? 1u : 0u);
}

// Value of a magnitude code as fp32 (exact).
template <class F>
__device__ __forceinline__ float code_value(uint32_t mag) {
  constexpr float STEP = pow2(1 - F::BIAS - F::MB);
  uint32_t e = mag >> F::MB;
  float normal = __uint_as_float((mag << (23 - F::MB)) + (static_cast<uint32_t>(127 - F::BIAS) << 23));
  float sub = static_cast<float>(mag) * STEP;
  return e ? normal : sub;
}

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014) and the
// 24-bit uniform drawn for element `idx`.
__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ float sr_uniform(uint64_t seed, uint64_t idx) {
  uint64_t h = splitmix64(seed ^ (0x9E3779B97F4A7C15ull * (idx + 1ull)));
  return static_cast<float>(static_cast<uint32_t>(h >> 40)) * (1.0f / 16777216.0f);
}

// Exchange a 32-bit value with the neighbouring lane (lane ^ 1) through DPP
// quad_perm [1,0,3,2].
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap_pair(float v) {
  return __uint_as_float(swap_pair(__float_as_uint(v)));
}

// Amax sentinel: bit patterns at or above this (with the sign cleared) are
// Inf or NaN.
constexpr uint32_t NONFINITE_BITS = 0x7F800000u;

}  // namespace mx
