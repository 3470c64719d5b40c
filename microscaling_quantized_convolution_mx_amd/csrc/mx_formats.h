// Device-side microscaling formats for gfx950.
//
// Element formats E2M1 / E2M3 / E4M3 and the E4M3 block scale of MicroQonv's
// NVFP4-style quantizer (arXiv 2609.28358, §II-D and §III-A), E3M2 (the FP6
// activations of MicroQonv+, §IV-D and Table VI) and the sign-less 3-bit
// E2M1 of post-ReLU activations (§VI-A).  Rounding works
// on the fp32 bit pattern: subnormal values by an exact power-of-two rescale
// and a round-to-integer, normal values by rounding the 23-bit mantissa to the
// format's width with carry into the exponent.  Both are the IEEE
// round-to-nearest-even of the value onto the format grid; values at or above
// the format maximum saturate to it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum { FMT_E2M1 = 1, FMT_E2M3 = 2, FMT_E4M3 = 3, FMT_UE2M1 = 4, FMT_E3M2 = 5 };

template <int FMT> struct Fmt;
template <> struct Fmt<FMT_E2M1> {
  static constexpr int MB = 1, BIAS = 1, SIGN = 3, BITS = 4, MAXCODE = 7;
  static constexpr float MAXV = 6.0f;
  static constexpr bool SIGNED = true;
};
// E2M1 magnitude without the sign bit (3-bit codes of post-ReLU activations,
// §VI-A): quantized like E2M1, a negative element keeps only its magnitude
template <> struct Fmt<FMT_UE2M1> {
  static constexpr int MB = 1, BIAS = 1, SIGN = 3, BITS = 3, MAXCODE = 7;
  static constexpr float MAXV = 6.0f;
  static constexpr bool SIGNED = false;
};
template <> struct Fmt<FMT_E2M3> {
  static constexpr int MB = 3, BIAS = 1, SIGN = 5, BITS = 6, MAXCODE = 31;
  static constexpr float MAXV = 7.5f;
  static constexpr bool SIGNED = true;
};
// FP6 with the wider range (max 28, subnormal step 1/16)
template <> struct Fmt<FMT_E3M2> {
  static constexpr int MB = 2, BIAS = 3, SIGN = 5, BITS = 6, MAXCODE = 31;
  static constexpr float MAXV = 28.0f;
  static constexpr bool SIGNED = true;
};
template <> struct Fmt<FMT_E4M3> {
  static constexpr int MB = 3, BIAS = 7, SIGN = 7, BITS = 8, MAXCODE = 126;
  static constexpr float MAXV = 448.0f;
  static constexpr bool SIGNED = true;
};
using ScaleFmt = Fmt<FMT_E4M3>;

// Bytes of one 8x8 block of codes.
template <int FMT> constexpr int block_bytes() { return Fmt<FMT>::BITS * 8; }

// 2^k as a float for small k (compile time).
__host__ __device__ constexpr float pow2(int k) {
  return k >= 0 ? float(1ull << k) : 1.0f / float(1ull << -k);
}

// Round-to-nearest-even magnitude code of v >= 0 (v may be +inf).  Both
// the subnormal and the normal candidate are computed and one is selected
// (no divergent branch).
template <class F>
__device__ __forceinline__ uint32_t rne_code(float v) {
  constexpr float MIN_NORMAL = pow2(1 - F::BIAS);
  // subnormal grid step 2^(1-BIAS-MB): code = nearest integer of v / step
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(fminf(v, MIN_NORMAL) * pow2(F::MB + F::BIAS - 1)));
  constexpr int SH = 23 - F::MB;
  uint32_t b = __float_as_uint(v);
  b += ((1u << (SH - 1)) - 1u) + ((b >> SH) & 1u);
  const uint32_t nor = (b >> SH) - static_cast<uint32_t>((127 - F::BIAS) << F::MB);
  const uint32_t c = v < MIN_NORMAL ? sub : nor;
  return v < F::MAXV ? c : static_cast<uint32_t>(F::MAXCODE);
}

// Stochastic rounding of v >= +0 (v may be +inf) with the uniform u / 2^24
// (u a 24-bit integer), passed as its complement ub = 2^24 - 1 - u: with
// lo <= v < hi the neighbouring grid points, round up iff
// u / 2^24 < (v - lo) / (hi - lo).  v is clamped to the format maximum
// first.  The grid step at v is 2^(e - MB) in the normal binade
// [2^e, 2^(e+1)) and the subnormal step 2^(1-BIAS-MB) below the smallest
// normal, so Q = v / step * 2^24 is an exact power-of-two rescale of v,
// below 2^(MB+25); lo / step is its integer part over 2^24 and the rule is
// u < X with X = Q - (lo / step) 2^24 in [0, 2^24).  For an integer u,
// u < X exactly when u < ceil(X), so with C = ceil(Q) = L 2^24 + F
// (0 <= F < 2^24) the rounded index lo / step + up is L + (u < F): where
// ceil(X) reaches 2^24 it has carried into L and F = 0.  u < F is the carry
// of F + ub out of the low 24 bits, so the index is (C + ub) >> 24.  Codes
// are that index plus (binade above the smallest) << MB: a round-up past the
// largest mantissa carries into the next binade.  Branch-free.
template <class F>
__device__ __forceinline__ uint32_t sr_code(float v, uint32_t ub) {
  constexpr int EMIN = 127 + 1 - F::BIAS;  // fp32 biased exponent of the smallest normal
  // v is +0 or positive (+inf and NaN lie above the maximum as bit
  // patterns): the clamp is the unsigned minimum of the bit patterns
  v = __uint_as_float(min(__float_as_uint(v), __float_as_uint(F::MAXV)));
  const uint32_t e = __builtin_amdgcn_ubfe(__float_as_uint(v), 23, 8);
  const uint32_t eb = e > static_cast<uint32_t>(EMIN) ? e - EMIN : 0u;  // binades above the smallest
  const float q = __builtin_amdgcn_ldexpf(v, (151 + F::MB - EMIN) - static_cast<int>(eb));
  // -ceil(Q) = floor(-Q) in one conversion (Q < 2^28: no saturation)
  int m;
  asm("v_cvt_flr_i32_f32 %0, -%1" : "=v"(m) : "v"(q));
  return (eb << F::MB) + ((ub - static_cast<uint32_t>(m)) >> 24);
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

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014), returned
// complemented (~z for the output z).  The stochastic-rounding uniform of
// element idx takes 24 bits of the output for counter idx / 2: bits 40..63
// for an even idx, bits 16..39 for an odd one; the same bits of the
// complement are 2^24 - 1 - u, the form sr_code takes.
__device__ __forceinline__ uint64_t splitmix64_not(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return ~(z ^ (z >> 31));
}
constexpr uint64_t kGolden64 = 0x9E3779B97F4A7C15ull;
// the complemented 24-bit uniforms of elements 2k, 2k+1 from
// gk = kGolden64 * (k + 1), taken from the two 32-bit halves of the output
// (a shift and a byte gather)
__device__ __forceinline__ void sr_ubar_pair(uint64_t seed, uint64_t gk, uint32_t& ub_even, uint32_t& ub_odd) {
  const uint64_t h = splitmix64_not(seed ^ gk);
  const uint32_t hi = static_cast<uint32_t>(h >> 32), lo = static_cast<uint32_t>(h);
  ub_even = hi >> 8;
  ub_odd = __builtin_amdgcn_perm(hi, lo, 0x0c040302u);  // bytes 2, 3 of lo and 0 of hi: bits 16..39
}
__device__ __forceinline__ uint32_t sr_ubar(uint64_t seed, uint64_t idx) {
  uint32_t ue, uo;
  sr_ubar_pair(seed, kGolden64 * ((idx >> 1) + 1ull), ue, uo);
  return (idx & 1ull) ? uo : ue;
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
