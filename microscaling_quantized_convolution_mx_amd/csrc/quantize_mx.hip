// Quantizer and dequantizer of the original microscaling format on square
// blocks: one E8M0 power-of-two scale per 32x32 block, no tensor scale
// (MicroQonv, arXiv 2609.28358, §II-D; §IV-B: the method holds for any block
// scale).  The shared exponent is the OCP MX one, floor(log2 amax_block)
// minus the exponent of the element format's largest value (2 for E2M1),
// clamped to [-127, 127]; an all-zero block takes code 0, a block holding
// Inf or NaN takes 0xFF (NaN) with all codes 0.  Each element is |x| / 2^e,
// one exact multiply by a power of two, rounded onto the E2M1 grid
// (nearest-even or stochastic, saturating), with the sign of x.
//
// Layouts (blocks in the channel-batch-first order of §IV-A):
//   ACT / GRAD  blocks [H][W][C/32][N/32], element (r, c) = (channel, sample)
//   WEIGHT      blocks [Kh][Kw][Co/32][Ci/32], element (r, c) = (co, ci)
// codes: a block is 32 rows of 16 bytes, element 2j of a row in the low
// nibble of byte j; scales: one E8M0 byte per block.
//
// One wave per block: lane l handles elements 4*(l%8) .. +3 of rows
// l/8 + 8q, q = 0..3, so that each memory instruction of the wave covers 8
// whole rows (8 x 128 bytes of fp32, 8 x 16 bytes of codes).  Unlike the
// two-level format there is no tensor-wide statistic, so the quantizer reads
// its source once.
#include "internal.h"
#include "mx_formats.h"

namespace mx {
namespace {

constexpr int kMxS = 32;            // block edge
constexpr int kMxWaves = 4;         // blocks per workgroup
constexpr int kMxEmaxE2M1 = 2;      // 6 = 1.5 * 2^2

struct MxDims {
  int64_t nblocks;
  int64_t n, c;        // ACT / GRAD: samples and channels
  int64_t ci, khkw;    // WEIGHT: input channels and taps
  int64_t cb, nb;      // ACT / GRAD: channel and sample blocks; WEIGHT: co and ci blocks
};

MxDims make_mx_dims(const Geom& g, mx_role role) {
  MxDims d{};
  if (role == MX_ROLE_WEIGHT) {
    d.ci = g.c_in;
    d.khkw = static_cast<int64_t>(g.k_h) * g.k_w;
    d.cb = g.c_out / kMxS;
    d.nb = g.c_in / kMxS;
    d.nblocks = d.khkw * d.cb * d.nb;
  } else {
    const bool act = role == MX_ROLE_ACT;
    d.c = act ? g.c_in : g.c_out;
    d.n = g.n;
    d.cb = d.c / kMxS;
    d.nb = g.n / kMxS;
    d.nblocks = (act ? static_cast<int64_t>(g.h) * g.w : static_cast<int64_t>(g.ho) * g.wo) * d.cb * d.nb;
  }
  return d;
}

// Source index of element (r, c0) of block b, and the stride between the
// lane's consecutive elements (1 for ACT / GRAD, Kh*Kw for WEIGHT).
template <int ROLE>
__device__ __forceinline__ int64_t mx_src(const MxDims& d, int64_t b, int r, int c0, int64_t& step) {
  const int64_t lo = b % d.nb, t = b / d.nb;
  const int64_t mid = t % d.cb, hi = t / d.cb;
  if constexpr (ROLE == MX_ROLE_WEIGHT) {
    // hi = tap, mid = co block, lo = ci block
    step = d.khkw;
    return ((mid * kMxS + r) * d.ci + lo * kMxS + c0) * d.khkw + hi;
  } else {
    // hi = spatial position, mid = channel block, lo = sample block
    step = 1;
    return (hi * d.c + mid * kMxS + r) * d.n + lo * kMxS + c0;
  }
}

// E8M0 code of the shared scale from the sign-cleared bits of the block
// maximum (NaN bits order above Inf above every finite value).
__device__ __forceinline__ uint32_t e8m0_code(uint32_t amax_bits) {
  if (amax_bits >= NONFINITE_BITS) return 0xFFu;
  if (amax_bits == 0u) return 0u;
  // floor(log2 amax): the exponent field, or the top set bit of a subnormal
  const int fl = amax_bits >= 0x00800000u ? static_cast<int>(amax_bits >> 23) - 127
                                          : (31 - __builtin_clz(amax_bits)) - 149;
  int e = fl - kMxEmaxE2M1;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return static_cast<uint32_t>(e + 127);
}

template <int ROLE, bool SR>
__global__ __launch_bounds__(kMxWaves * 64) void k_quantize_mx(const float* __restrict__ src, const MxDims d,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales, float* tensor_scale,
                                                                uint64_t seed) {
  using F = Fmt<FMT_E2M1>;
  const int lane = threadIdx.x & 63;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kMxWaves + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = 1.0f;  // no tensor scale
  if (b >= d.nblocks) return;  // whole waves
  const int r0 = lane >> 3, c0 = (lane & 7) * 4;
  int64_t step;
  int64_t s0[4];  // source index of element (r0 + 8q, c0)
#pragma unroll
  for (int q = 0; q < 4; ++q) s0[q] = mx_src<ROLE>(d, b, r0 + 8 * q, c0, step);

  float x[16];  // x[4q + j] = element (r0 + 8q, c0 + j)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * q + j] = src[s0[q] + j * step];
    } else {
      const float4 v = *reinterpret_cast<const float4*>(src + s0[q]);
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = max(m, __float_as_uint(x[j]) & 0x7FFFFFFFu);
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  const uint32_t code = e8m0_code(m);
  // 1 / 2^e = 2^(127 - code): a normal fp32 for every code a finite block
  // can take (code <= 125 + 2 at most)
  const float inv = __uint_as_float((254u - min(code, 253u)) << 23);
  const bool nonfinite = code == 0xFFu;

  uint32_t w[4] = {0u, 0u, 0u, 0u};  // 4 codes (16 bits) of each of the lane's rows
  if constexpr (!SR) {
    // the hardware conversion rounds to nearest even and keeps the sign of
    // its input; the magnitude is clamped to the format maximum first
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float sv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = nonfinite ? 0.0f : fminf(fabsf(x[4 * q + j]) * inv, F::MAXV);
        sv[j] = __builtin_copysignf(v, nonfinite ? 1.0f : x[4 * q + j]);
      }
      uint32_t t = 0;
      t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, sv[0], sv[1], 1.0f, 0);
      t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, sv[2], sv[3], 1.0f, 1);
      w[q] = t;
    }
  } else {
    uint32_t ub[16];  // complemented SR uniforms
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ub[4 * q + j] = sr_ubar(seed, static_cast<uint64_t>(s0[q] + j * step));
      } else {
        // 4 consecutive elements from an even index: 2 draws
        const uint64_t gk = kGolden64 * (static_cast<uint64_t>(s0[q] >> 1) + 1ull);
        sr_ubar_pair(seed, gk, ub[4 * q], ub[4 * q + 1]);
        sr_ubar_pair(seed, gk + kGolden64, ub[4 * q + 2], ub[4 * q + 3]);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t mag = nonfinite ? 0u : sr_code<F>(fabsf(x[j]) * inv, ub[j]);
      const uint32_t sign = nonfinite ? 0u : (__float_as_uint(x[j]) >> 31);
      w[j >> 2] |= (mag | (sign << F::SIGN)) << (4 * (j & 3));
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint16_t*>(codes + b * 512 + (r0 + 8 * q) * 16 + (lane & 7) * 2) = static_cast<uint16_t>(w[q]);
  if (lane == 0) scales[b] = static_cast<uint8_t>(code);
}

template <int ROLE>
__global__ __launch_bounds__(kMxWaves * 64) void k_dequantize_mx(const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales, const MxDims d,
                                                                  float* __restrict__ dst) {
  using F = Fmt<FMT_E2M1>;
  const int lane = threadIdx.x & 63;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * kMxWaves + (threadIdx.x >> 6);
  if (b >= d.nblocks) return;
  const int r0 = lane >> 3, c0 = (lane & 7) * 4;
  int64_t step;
  int64_t s0[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) s0[q] = mx_src<ROLE>(d, b, r0 + 8 * q, c0, step);
  const uint32_t code = scales[b];
  // 2^(code - 127): 2^-127 is the fp32 subnormal 0x00400000; 0xFF is NaN
  const float scale = code == 0xFFu ? __uint_as_float(0x7FC00000u)
                                    : (code == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = *reinterpret_cast<const uint16_t*>(codes + b * 512 + (r0 + 8 * q) * 16 + (lane & 7) * 2);
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c = (w >> (4 * j)) & 0xFu;
      const float v = code_value<F>(c & 7u) * scale;  // exact: a multiple of 2^-128 within range
      y[j] = (c >> 3) ? -v : v;
    }
    if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[s0[q] + j * step] = y[j];
    } else {
      *reinterpret_cast<float4*>(dst + s0[q]) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}

template <int ROLE>
void launch_q_mx(const MxDims& d, const float* src, const mx_qtensor* dst, bool sr, uint64_t seed, hipStream_t s) {
  const unsigned wgs = static_cast<unsigned>((d.nblocks + kMxWaves - 1) / kMxWaves);
  uint8_t* codes = static_cast<uint8_t*>(dst->codes);
  if (wgs == 0) {
    // still report the (absent) tensor scale
    hipLaunchKernelGGL((k_quantize_mx<ROLE, false>), dim3(1), dim3(64), 0, s, src, d, codes, dst->scales,
                       dst->tensor_scale, seed);
    return;
  }
  if (sr)
    hipLaunchKernelGGL((k_quantize_mx<ROLE, true>), dim3(wgs), dim3(kMxWaves * 64), 0, s, src, d, codes,
                       dst->scales, dst->tensor_scale, seed);
  else
    hipLaunchKernelGGL((k_quantize_mx<ROLE, false>), dim3(wgs), dim3(kMxWaves * 64), 0, s, src, d, codes,
                       dst->scales, dst->tensor_scale, seed);
}

template <int ROLE>
void launch_dq_mx(const MxDims& d, const mx_qtensor* q, float* dst, hipStream_t s) {
  const unsigned wgs = static_cast<unsigned>((d.nblocks + kMxWaves - 1) / kMxWaves);
  if (wgs == 0) return;
  hipLaunchKernelGGL((k_dequantize_mx<ROLE>), dim3(wgs), dim3(kMxWaves * 64), 0, s,
                     static_cast<const uint8_t*>(q->codes), q->scales, d, dst);
}

}  // namespace

hipError_t launch_quantize_mx(const Geom& g, mx_role role, const float* src, const mx_qtensor* dst,
                              mx_round rounding, uint64_t seed, hipStream_t s) {
  const MxDims d = make_mx_dims(g, role);
  const bool sr = rounding == MX_SR;
  switch (role) {
    case MX_ROLE_ACT: launch_q_mx<MX_ROLE_ACT>(d, src, dst, sr, seed, s); break;
    case MX_ROLE_GRAD: launch_q_mx<MX_ROLE_GRAD>(d, src, dst, sr, seed, s); break;
    default: launch_q_mx<MX_ROLE_WEIGHT>(d, src, dst, sr, seed, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_mx(const Geom& g, mx_role role, const mx_qtensor* q, float* dst, hipStream_t s) {
  const MxDims d = make_mx_dims(g, role);
  switch (role) {
    case MX_ROLE_ACT: launch_dq_mx<MX_ROLE_ACT>(d, q, dst, s); break;
    case MX_ROLE_GRAD: launch_dq_mx<MX_ROLE_GRAD>(d, q, dst, s); break;
    default: launch_dq_mx<MX_ROLE_WEIGHT>(d, q, dst, s); break;
  }
  return hipGetLastError();
}

}  // namespace mx
