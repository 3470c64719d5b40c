// Quantization of convolution tensors into 8x8 microscaling blocks, and the
// inverse (fake-quantized fp32 values).
//
// MicroQonv (arXiv 2609.28358) quantizes every tensor of a convolution layer
// once (§IV-C), in square 8x8 blocks laid out channel-batch-first (§IV-A,
// §IV-B), with NVFP4-style two-level scaling: an fp32 per-tensor scale from
// the tensor amax and an E4M3 per-block scale (§III-A).
//
// Work decomposition (HBM-bound): a pair of neighbouring lanes owns one 8x8
// block; each lane holds 4 of the 8 columns of all 8 rows.  For activations
// and gradients a block row is 8 consecutive batch elements (32 bytes), so a
// wavefront (32 blocks) streams whole rows of the (C, N) plane with 16-byte
// loads.  The block amax and the packed code rows are exchanged between the
// two lanes with one DPP move each; the codes leave as 16-byte stores.
#include "internal.h"
#include "mx_formats.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerWG = kThreads / 2;

struct QDims {
  int64_t nblocks;
  int32_t d0, d1, d2, d3;  // ACT/GRAD: H, W, C, N   WEIGHT: Co, Ci, Kh, Kw
};

__global__ void k_amax_zero(uint32_t* amax_bits) {
  if (threadIdx.x == 0) *amax_bits = 0u;
}

// max |x| as the unsigned max of the bit patterns with the sign cleared:
// exact, order-independent, and Inf/NaN come out at or above 0x7F800000.
__global__ __launch_bounds__(kThreads) void k_amax(const uint4* __restrict__ src, int64_t n4,
                                                   uint32_t* amax_bits) {
  uint32_t m = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    m = max(m, max(max(v0.x & 0x7FFFFFFFu, v0.y & 0x7FFFFFFFu), max(v0.z & 0x7FFFFFFFu, v0.w & 0x7FFFFFFFu)));
    m = max(m, max(max(v1.x & 0x7FFFFFFFu, v1.y & 0x7FFFFFFFu), max(v1.z & 0x7FFFFFFFu, v1.w & 0x7FFFFFFFu)));
    m = max(m, max(max(v2.x & 0x7FFFFFFFu, v2.y & 0x7FFFFFFFu), max(v2.z & 0x7FFFFFFFu, v2.w & 0x7FFFFFFFu)));
    m = max(m, max(max(v3.x & 0x7FFFFFFFu, v3.y & 0x7FFFFFFFu), max(v3.z & 0x7FFFFFFFu, v3.w & 0x7FFFFFFFu)));
  }
  for (; i < n4; i += stride) {
    uint4 v = src[i];
    m = max(m, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
    for (int k = 1; k < kThreads / 64; ++k) r = max(r, part[k]);
    atomicMax(amax_bits, r);
  }
}

// fp32 source offset of element (r, c) of a block: base + r*row + c*col.
// The block coordinates are decoded once per lane (32-bit arithmetic: block
// counts are below 2^31).
struct BlockAddr {
  int64_t base, row, col;
};

template <int ROLE>
__device__ __forceinline__ BlockAddr block_addr(const QDims& d, int64_t blk) {
  const uint32_t b = static_cast<uint32_t>(blk);
  BlockAddr a;
  if constexpr (ROLE == MX_ROLE_WEIGHT) {
    const uint32_t cib_n = static_cast<uint32_t>(d.d1) >> 3, cob_n = static_cast<uint32_t>(d.d0) >> 3;
    const uint32_t khkw = static_cast<uint32_t>(d.d2 * d.d3);
    uint32_t t = b / cib_n;
    const uint32_t cib = b - t * cib_n;
    const uint32_t t2 = t / cob_n;
    const uint32_t cob = t - t2 * cob_n;
    const uint32_t kh = t2 / static_cast<uint32_t>(d.d3), kw = t2 - kh * static_cast<uint32_t>(d.d3);
    a.base = (static_cast<int64_t>(cob) * 8 * d.d1 + cib * 8) * khkw + kh * d.d3 + kw;
    a.row = static_cast<int64_t>(d.d1) * khkw;
    a.col = khkw;
  } else {
    const uint32_t nb_n = static_cast<uint32_t>(d.d3) >> 3, cb_n = static_cast<uint32_t>(d.d2) >> 3;
    const uint32_t t = b / nb_n;
    const uint32_t nb = b - t * nb_n;
    const uint32_t p = t / cb_n;
    const uint32_t cb = t - p * cb_n;
    a.base = (static_cast<int64_t>(p) * d.d2 + cb * 8) * d.d3 + nb * 8;
    a.row = d.d3;
    a.col = 1;
  }
  return a;
}

// Write this lane's half of a block whose 8 code rows are split between the
// lane pair: row_bits[r] holds the 4 codes of this lane's column half.
template <int FMT>
__device__ __forceinline__ void store_block_codes(uint8_t* __restrict__ codes, int64_t blk, int half,
                                                  const uint32_t (&rb)[8], bool valid) {
  if constexpr (FMT == FMT_E2M1) {
    // row = 4 bytes: low 16 bits from the even lane, high 16 bits from the odd
    const uint32_t s0 = half ? (rb[0] | (rb[1] << 16)) : (rb[4] | (rb[5] << 16));
    const uint32_t s1 = half ? (rb[2] | (rb[3] << 16)) : (rb[6] | (rb[7] << 16));
    const uint32_t r0 = swap_pair(s0), r1 = swap_pair(s1);
    uint4 out;
    if (half == 0) {
      out.x = rb[0] | ((r0 & 0xFFFFu) << 16);
      out.y = rb[1] | (r0 & 0xFFFF0000u);
      out.z = rb[2] | ((r1 & 0xFFFFu) << 16);
      out.w = rb[3] | (r1 & 0xFFFF0000u);
    } else {
      out.x = (r0 & 0xFFFFu) | (rb[4] << 16);
      out.y = (r0 >> 16) | (rb[5] << 16);
      out.z = (r1 & 0xFFFFu) | (rb[6] << 16);
      out.w = (r1 >> 16) | (rb[7] << 16);
    }
    if (valid) *reinterpret_cast<uint4*>(codes + blk * 32 + half * 16) = out;
  } else if constexpr (FMT == FMT_E4M3) {
    // row = 8 bytes: first dword from the even lane, second from the odd
    uint32_t rcv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rcv[i] = swap_pair(half ? rb[i] : rb[4 + i]);
    uint4 o0, o1;
    if (half == 0) {
      o0 = make_uint4(rb[0], rcv[0], rb[1], rcv[1]);
      o1 = make_uint4(rb[2], rcv[2], rb[3], rcv[3]);
    } else {
      o0 = make_uint4(rcv[0], rb[4], rcv[1], rb[5]);
      o1 = make_uint4(rcv[2], rb[6], rcv[3], rb[7]);
    }
    if (valid) {
      uint4* p = reinterpret_cast<uint4*>(codes + blk * 64 + half * 32);
      p[0] = o0;
      p[1] = o1;
    }
  } else {
    // E2M3: row = 48 bits (6 bytes), low 24 bits from the even lane
    const int base = half ? 0 : 4;
    const uint32_t a0 = rb[base], a1 = rb[base + 1], a2 = rb[base + 2], a3 = rb[base + 3];
    const uint32_t w0 = a0 | (a1 << 24), w1 = (a1 >> 8) | (a2 << 16), w2 = (a2 >> 16) | (a3 << 8);
    const uint32_t v0 = swap_pair(w0), v1 = swap_pair(w1), v2 = swap_pair(w2);
    uint32_t o[4];  // partner's four 24-bit row halves
    o[0] = v0 & 0xFFFFFFu;
    o[1] = (v0 >> 24) | ((v1 & 0xFFFFu) << 8);
    o[2] = (v1 >> 16) | ((v2 & 0xFFu) << 16);
    o[3] = v2 >> 8;
    uint64_t row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t lo = half ? o[i] : rb[i];
      const uint64_t hi = half ? rb[4 + i] : o[i];
      row[i] = lo | (hi << 24);
    }
    const uint64_t q0 = row[0] | (row[1] << 48);
    const uint64_t q1 = (row[1] >> 16) | (row[2] << 32);
    const uint64_t q2 = (row[2] >> 32) | (row[3] << 16);
    if (valid) {
      uint2* p = reinterpret_cast<uint2*>(codes + blk * 48 + half * 24);
      p[0] = make_uint2(static_cast<uint32_t>(q0), static_cast<uint32_t>(q0 >> 32));
      p[1] = make_uint2(static_cast<uint32_t>(q1), static_cast<uint32_t>(q1 >> 32));
      p[2] = make_uint2(static_cast<uint32_t>(q2), static_cast<uint32_t>(q2 >> 32));
    }
  }
}

template <int FMT, int ROLE, bool SR>
__global__ __launch_bounds__(kThreads) void k_quantize(const float* __restrict__ src,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       float* __restrict__ tensor_scale,
                                                       const float* __restrict__ amax, QDims d,
                                                       uint64_t seed) {
  using F = Fmt<FMT>;
  const int half = threadIdx.x & 1;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * kBlocksPerWG + (threadIdx.x >> 1);
  const bool valid = blk < d.nblocks;
  const uint32_t ab = __float_as_uint(*amax) & 0x7FFFFFFFu;

  if (ab >= NONFINITE_BITS) {  // non-finite input: T = NaN, scales 0x7F, codes 0
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = __uint_as_float(0x7FC00000u);
    const uint32_t zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    store_block_codes<FMT>(codes, blk, half, zero, valid);
    if (valid && half == 0) scales[blk] = 0x7F;
    return;
  }
  const float T = __uint_as_float(ab) / (448.0f * F::MAXV);
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = T;

  float x[8][4];
  const BlockAddr ad = block_addr<ROLE>(d, valid ? blk : 0);
  const int64_t base = ad.base + half * 4 * ad.col;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[r][j] = valid ? src[base + r * ad.row + j * ad.col] : 0.0f;
    } else {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (valid) v = *reinterpret_cast<const float4*>(src + base + r * ad.row);
      x[r][0] = v.x;
      x[r][1] = v.y;
      x[r][2] = v.z;
      x[r][3] = v.w;
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) am = fmaxf(am, fabsf(x[r][j]));
  am = fmaxf(am, swap_pair(am));

  const float den = F::MAXV * T;
  const float braw = (T == 0.0f) ? 0.0f : am / den;
  const uint32_t bcode = rne_code<ScaleFmt>(braw);
  const float B = code_value<ScaleFmt>(bcode);
  const float dd = B * T;

  uint32_t rb[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = (dd == 0.0f) ? 0.0f : fabsf(x[r][j]) / dd;
      uint32_t mag;
      if constexpr (SR) {
        const int64_t idx = base + r * ad.row + j * ad.col;
        mag = sr_code<F>(v, sr_uniform(seed, static_cast<uint64_t>(idx)));
      } else {
        mag = rne_code<F>(v);
      }
      const uint32_t code = mag | ((__float_as_uint(x[r][j]) >> 31) << F::SIGN);
      bits |= code << (F::BITS * j);
    }
    rb[r] = bits;
  }
  store_block_codes<FMT>(codes, blk, half, rb, valid);
  if (valid && half == 0) scales[blk] = static_cast<uint8_t>(bcode);
}

// Code of element (r, c) from the 32-bit words of one block.
template <int FMT>
__device__ __forceinline__ uint32_t get_code(const uint32_t* w, int r, int c) {
  constexpr int BITS = Fmt<FMT>::BITS;
  const int bit = (r * 8 + c) * BITS;
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

template <int FMT, int ROLE>
__global__ __launch_bounds__(kThreads) void k_dequantize(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ tensor_scale,
                                                         float* __restrict__ dst, QDims d) {
  using F = Fmt<FMT>;
  constexpr int BYTES = block_bytes<FMT>();
  const int half = threadIdx.x & 1;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * kBlocksPerWG + (threadIdx.x >> 1);
  if (blk >= d.nblocks) return;
  uint32_t w[BYTES / 4];
  const uint4* p = reinterpret_cast<const uint4*>(codes + blk * BYTES);
#pragma unroll
  for (int i = 0; i < BYTES / 16; ++i) {
    const uint4 v = p[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  const uint32_t sb = scales[blk];
  const float B = (sb == 0x7Fu) ? __uint_as_float(0x7FC00000u) : code_value<ScaleFmt>(sb);
  const float T = *tensor_scale;
  const BlockAddr ad = block_addr<ROLE>(d, blk);
  const int64_t base = ad.base + half * 4 * ad.col;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t code = get_code<FMT>(w, r, half * 4 + j);
      const float g = code_value<F>(code & ((1u << F::SIGN) - 1u));
      const float gb = g * B;
      float v = gb * T;
      if ((code >> F::SIGN) & 1u) v = -v;
      o[j] = v;
    }
    if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[base + r * ad.row + j * ad.col] = o[j];
    } else {
      *reinterpret_cast<float4*>(dst + base + r * ad.row) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

QDims make_qdims(const Geom& g, mx_role role) {
  QDims d;
  d.nblocks = role_nblocks(g, role);
  if (role == MX_ROLE_WEIGHT) {
    d.d0 = g.c_out; d.d1 = g.c_in; d.d2 = g.k_h; d.d3 = g.k_w;
  } else if (role == MX_ROLE_ACT) {
    d.d0 = g.h; d.d1 = g.w; d.d2 = g.c_in; d.d3 = g.n;
  } else {
    d.d0 = g.ho; d.d1 = g.wo; d.d2 = g.c_out; d.d3 = g.n;
  }
  return d;
}

template <int FMT, int ROLE>
void launch_q(const QDims& d, const float* src, const mx_qtensor* q, bool sr, uint64_t seed,
              hipStream_t s) {
  // at least one workgroup, so that an empty tensor still publishes T
  unsigned grid = static_cast<unsigned>((d.nblocks + kBlocksPerWG - 1) / kBlocksPerWG);
  if (grid == 0) grid = 1;
  auto* codes = static_cast<uint8_t*>(q->codes);
  if (sr)
    hipLaunchKernelGGL((k_quantize<FMT, ROLE, true>), dim3(grid), dim3(kThreads), 0, s, src, codes,
                       q->scales, q->tensor_scale, q->amax, d, seed);
  else
    hipLaunchKernelGGL((k_quantize<FMT, ROLE, false>), dim3(grid), dim3(kThreads), 0, s, src, codes,
                       q->scales, q->tensor_scale, q->amax, d, seed);
}

template <int FMT>
void launch_q_role(mx_role role, const QDims& d, const float* src, const mx_qtensor* q, bool sr,
                   uint64_t seed, hipStream_t s) {
  if (role == MX_ROLE_ACT) launch_q<FMT, MX_ROLE_ACT>(d, src, q, sr, seed, s);
  else if (role == MX_ROLE_GRAD) launch_q<FMT, MX_ROLE_GRAD>(d, src, q, sr, seed, s);
  else launch_q<FMT, MX_ROLE_WEIGHT>(d, src, q, sr, seed, s);
}

template <int FMT, int ROLE>
void launch_dq(const QDims& d, const mx_qtensor* q, float* dst, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>((d.nblocks + kBlocksPerWG - 1) / kBlocksPerWG);
  if (grid == 0) return;
  hipLaunchKernelGGL((k_dequantize<FMT, ROLE>), dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(q->codes), q->scales, q->tensor_scale, dst, d);
}

template <int FMT>
void launch_dq_role(mx_role role, const QDims& d, const mx_qtensor* q, float* dst, hipStream_t s) {
  if (role == MX_ROLE_ACT) launch_dq<FMT, MX_ROLE_ACT>(d, q, dst, s);
  else if (role == MX_ROLE_GRAD) launch_dq<FMT, MX_ROLE_GRAD>(d, q, dst, s);
  else launch_dq<FMT, MX_ROLE_WEIGHT>(d, q, dst, s);
}

}  // namespace

hipError_t launch_quantize(const Geom& g, mx_role role, const float* src, const mx_qtensor* dst,
                           mx_round rounding, uint64_t seed, int amax_given, hipStream_t s) {
  const QDims d = make_qdims(g, role);
  const int64_t numel = role_numel(g, role);
  auto* amax_bits = reinterpret_cast<uint32_t*>(dst->amax);
  if (!amax_given) {
    hipLaunchKernelGGL(k_amax_zero, dim3(1), dim3(64), 0, s, amax_bits);
    const int64_t n4 = numel / 4;
    if (n4 > 0) {
      int64_t wgs = (n4 + kThreads * 4 - 1) / (kThreads * 4);
      if (wgs > 4096) wgs = 4096;
      hipLaunchKernelGGL(k_amax, dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
                         reinterpret_cast<const uint4*>(src), n4, amax_bits);
    }
  }
  const bool sr = rounding == MX_SR;
  switch (g.fmt) {
    case FMT_E2M1: launch_q_role<FMT_E2M1>(role, d, src, dst, sr, seed, s); break;
    case FMT_E2M3: launch_q_role<FMT_E2M3>(role, d, src, dst, sr, seed, s); break;
    default: launch_q_role<FMT_E4M3>(role, d, src, dst, sr, seed, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const Geom& g, mx_role role, const mx_qtensor* q, float* dst,
                             hipStream_t s) {
  const QDims d = make_qdims(g, role);
  switch (g.fmt) {
    case FMT_E2M1: launch_dq_role<FMT_E2M1>(role, d, q, dst, s); break;
    case FMT_E2M3: launch_dq_role<FMT_E2M3>(role, d, q, dst, s); break;
    default: launch_dq_role<FMT_E4M3>(role, d, q, dst, s); break;
  }
  return hipGetLastError();
}

}  // namespace mx
