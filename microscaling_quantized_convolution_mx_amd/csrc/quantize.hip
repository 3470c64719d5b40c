// Quantization of convolution tensors into 8x8 microscaling blocks, and the
// inverse (fake-quantized fp32 values).
//
// MicroQonv (arXiv 2609.28358) quantizes every tensor of a convolution layer
// once (§IV-C), in square 8x8 blocks laid out channel-batch-first (§IV-A,
// §IV-B), with NVFP4-style two-level scaling: an fp32 per-tensor scale from
// the tensor amax and an E4M3 per-block scale (§III-A).
//
// Two kernels per tensor, no atomics:
//   k_amax_part       each workgroup writes the max |x| of its grid-stride
//                     share as one 32-bit partial into a scratch tail behind
//                     the block scales (the scales buffer is sized for it),
//                     with a flag bit for magnitudes below 2^-64;
//   k_quantize_wide   activations and gradients: every wave reduces the
//                     partials to the tensor amax and T, each workgroup
//                     tabulates dd = B T and RN(1 / dd) for the 127 block-scale
//                     codes in LDS, then quantizes 32 blocks per iteration
//                     (the next 32 in flight), two lanes per block, each row
//                     load of a wave 1 KiB contiguous;
//   k_quantize        weights (strided rows): the same arithmetic with one
//                     lane per block row, 8 blocks per wave iteration.
// Tensors of at most kOneBlocks blocks take k_quantize in a single
// workgroup that computes the amax itself: one launch.
#include "internal.h"
#include "mx_formats.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerWG = kThreads / 64;  // 8-block groups per workgroup iteration
constexpr int kQuantMaxWGs = 2048;

struct QDims {
  int64_t nblocks;
  int32_t d0, d1, d2, d3;  // ACT/GRAD: H, W, C, N   WEIGHT: Co, Ci, Kh, Kw
  // ACT/GRAD: division by the batch-block and channel-block counts as
  // mulhi(x, m) >> s (m = 0: divisor 1)
  uint32_t m_nb, m_cb;
  int32_t s_nb, s_cb;
};

// Magic multiplier for x / d with x < 2^31: m = ceil(2^(31+l) / d),
// l = ceil(log2 d), so that floor(x / d) = floor(x m / 2^(31+l)).
inline void magic_div(uint32_t d, uint32_t& m, int32_t& sh) {
  if (d <= 1) { m = 0; sh = 0; return; }
  int l = 0;
  while ((1ull << l) < d) ++l;
  m = static_cast<uint32_t>(((1ull << (31 + l)) + d - 1) / d);
  sh = l - 1;  // applied to the high 32 bits of the 64-bit product
}
__device__ __forceinline__ uint32_t magic_quot(uint32_t x, uint32_t m, int32_t sh) {
  return m == 0u ? x : (__umulhi(x, m) >> sh);
}

__device__ __forceinline__ uint32_t absbits(uint32_t v) { return v & 0x7FFFFFFFu; }

// Streaming 16-byte load with the nontemporal hint: the source of a
// quantization pass is read once per pass, and on this GPU the hinted loads
// sustain ~15% more read bandwidth than plain ones.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_stream(const float* p) {
  const uint4 v = load_stream(reinterpret_cast<const uint4*>(p));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ uint32_t max4(uint4 v) {
  return max(max(absbits(v.x), absbits(v.y)), max(absbits(v.z), absbits(v.w)));
}

// Max |x| as the unsigned max of the bit patterns with the sign cleared:
// exact, order-independent, and Inf/NaN come out at or above 0x7F800000.
// Workgroup b writes its share's max to part[b]; every workgroup writes.
// Bit 31 of part[b] (never set in a max of cleared sign bits) flags a
// nonzero element of the share below 2^-64 in magnitude: a tensor with no
// flag and amax <= 2^34 has no element that the quantizer's reciprocal
// quotient must divide instead (k_quantize_wide).
// 16 waves per workgroup: with at most kAmaxMaxPartials workgroups, 8 loads
// of 16 bytes in flight per lane still make 128 KiB per CU.
constexpr int kAmaxThreads = 1024;
constexpr uint32_t kPartTiny = 0x80000000u;
// 2 bits(|x|) - 1 (a zero wraps to the maximum) and its bound for 2^-64
__device__ __forceinline__ uint32_t tiny_key(uint32_t v) { return (v << 1) - 1u; }
constexpr uint32_t kTinyKey64 = (0x1F800000u << 1) - 1u;
__device__ __forceinline__ uint32_t min4key(uint4 v) {
  return min(min(tiny_key(v.x), tiny_key(v.y)), min(tiny_key(v.z), tiny_key(v.w)));
}
__global__ __launch_bounds__(kAmaxThreads) void k_amax_part(const uint4* __restrict__ src, int64_t n4,
                                                            uint32_t* __restrict__ part) {
  uint32_t m = 0, mk = ~0u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kAmaxThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kAmaxThreads + threadIdx.x;
  for (; i + 7 * stride < n4; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load_stream(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m = max(m, max4(v[k]));
      mk = min(mk, min4key(v[k]));
    }
  }
  for (; i < n4; i += stride) {
    const uint4 v = load_stream(src + i);
    m = max(m, max4(v));
    mk = min(mk, min4key(v));
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  __shared__ uint32_t wmax[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  const int tiny = __syncthreads_or(mk < kTinyKey64);
  if (threadIdx.x == 0) {
    uint32_t r = wmax[0];
    for (int k = 1; k < kAmaxThreads / 64; ++k) r = max(r, wmax[k]);
    part[blockIdx.x] = r | (tiny ? kPartTiny : 0u);
  }
}

// fp32 source offset of element (r, c) of a block: base + r*row + c*col.
// The block coordinates are decoded with 32-bit arithmetic (block counts are
// below 2^31).
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
    const uint32_t t = magic_quot(b, d.m_nb, d.s_nb);
    const uint32_t nb = b - t * nb_n;
    const uint32_t p = magic_quot(t, d.m_cb, d.s_cb);
    const uint32_t cb = t - p * cb_n;
    a.base = (static_cast<int64_t>(p) * d.d2 + cb * 8) * d.d3 + nb * 8;
    a.row = d.d3;
    a.col = 1;
  }
  return a;
}

// DPP moves inside a group of 8 lanes: quad_perm [1,0,3,2], [2,3,0,1] and
// row_half_mirror (lane i <-> 7-i).
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  return v;
}

// Store one code row (8 codes, `lo` = bits 0..31, `hi` = bits 32..63) of
// block `blk`; row r of a block starts at bit 8*BITS*r of the block.
template <int FMT>
__device__ __forceinline__ void store_row(uint8_t* __restrict__ codes, int64_t blk, int r, uint32_t lo,
                                          uint32_t hi, bool valid) {
  if constexpr (FMT == FMT_E2M1) {
    if (valid) *reinterpret_cast<uint32_t*>(codes + blk * 32 + r * 4) = lo;
  } else if constexpr (FMT == FMT_E4M3) {
    if (valid) *reinterpret_cast<uint2*>(codes + blk * 64 + r * 8) = make_uint2(lo, hi);
  } else if constexpr (FMT == FMT_UE2M1) {
    // 24-bit rows: the first lane of each quad (rows 4q..4q+3) writes them as
    // three words at byte 12q of the 24-byte block
    const int lane = threadIdx.x & 63;
    const uint32_t r1 = static_cast<uint32_t>(__shfl(static_cast<int>(lo), lane + 1));
    const uint32_t r2 = static_cast<uint32_t>(__shfl(static_cast<int>(lo), lane + 2));
    const uint32_t r3 = static_cast<uint32_t>(__shfl(static_cast<int>(lo), lane + 3));
    if (valid && (r & 3) == 0) {
      uint32_t* q = reinterpret_cast<uint32_t*>(codes + blk * 24 + (r >> 2) * 12);
      q[0] = lo | (r1 << 24);
      q[1] = (r1 >> 8) | (r2 << 16);
      q[2] = (r2 >> 16) | (r3 << 8);
    }
  } else {
    // 48-bit rows: the even lane of each pair writes both rows (12 bytes)
    const uint32_t plo = swap_pair(lo), phi = swap_pair(hi);
    if (valid && (r & 1) == 0) {
      uint32_t* q = reinterpret_cast<uint32_t*>(codes + blk * 48 + (r >> 1) * 12);
      q[0] = lo;
      q[1] = (hi & 0xFFFFu) | (plo << 16);
      q[2] = (plo >> 16) | (phi << 16);
    }
  }
}

typedef short short2v __attribute__((ext_vector_type(2)));

// RN(a / b) from y = RN(1 / b) with two fused multiply-adds: the residual
// a - b q of q = RN(a y) is exact and RN(q + (a - b q) y) = RN(a / b)
// (Markstein, IBM J. Res. Dev. 34(1), 1990) as long as nothing under- or
// overflows.  That holds when b is in [2^-125, 2^125], a is 0 or at least
// max(2^-100, b 2^-98) (so that q >= 2^-100 and the residual is not
// subnormal) and a / b is below 2^100; callers check the first two and
// divide otherwise, the third holds by construction at every call.
__device__ __forceinline__ float div_by_recip(float a, float b, float y) {
  const float q = a * y;
  return __builtin_fmaf(__builtin_fmaf(-q, b, a), y, q);
}

// E4M3 round-to-nearest-even code of b >= 0 through the hardware packed
// conversion (identical to rne_code<ScaleFmt> once b is clamped to 448).
__device__ __forceinline__ uint32_t rne_e4m3_hw(float b) {
  const short2v w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(short2v{0, 0}, fminf(b, 448.0f), 0.0f, 1.0f, false);
  return static_cast<uint32_t>(static_cast<uint16_t>(w.x)) & 0xFFu;
}

// The 8 source values of code row r of block blk (blk clamped to block 0
// when past the tensor: always loaded, never stored).
template <int ROLE>
struct RowIn {
  float x[8];
  int64_t rowbase, col;
  __device__ __forceinline__ void load(const float* __restrict__ src, const QDims& d, int64_t blk, int r) {
    const BlockAddr ad = block_addr<ROLE>(d, blk);
    rowbase = ad.base + r * ad.row;
    col = ad.col;
    if (d.nblocks == 0) {  // an empty tensor: nothing to read
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.0f;
      return;
    }
    if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = src[rowbase + j * ad.col];
    } else {
      const float4 v0 = load_stream(src + rowbase);
      const float4 v1 = load_stream(src + rowbase + 4);
      x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
      x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    }
  }
};

// One entry of the per-workgroup table of block-scale codes (below).
struct ScaleEntry {
  float dd, y;
  uint32_t tiny, all_slow;
};

// ONE: a single 1024-thread workgroup that also computes the amax (nparts
// >= 0) over the whole tensor first, for tensors of at most kOneBlocks
// blocks (up to 4 loads of 16 bytes per thread): one launch instead of two.
// Beyond 256 blocks one workgroup is slower than the two launches (weights,
// whose rows are strided gathers, most of all).
constexpr int kOneThreads = 1024;
constexpr int64_t kOneBlocks = 256;  // at most 2 groups per wave
template <int FMT, int ROLE, bool SR, bool ONE>
__global__ __launch_bounds__(ONE ? kOneThreads : kThreads) void k_quantize(const float* __restrict__ src,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       float* __restrict__ tensor_scale,
                                                       float* __restrict__ amax, const uint32_t* __restrict__ part,
                                                       int nparts, QDims d, uint64_t seed) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int r = lane & 7;
  const int64_t ngroups = (d.nblocks + 7) >> 3;
  const int64_t gstride = ONE ? kOneThreads / 64 : static_cast<int64_t>(gridDim.x) * kGroupsPerWG;
  int64_t grp = (ONE ? 0 : static_cast<int64_t>(blockIdx.x) * kGroupsPerWG) + (threadIdx.x >> 6);
  auto group_blk = [&](int64_t g) {
    const int64_t b = g * 8 + (lane >> 3);
    return b < d.nblocks ? b : int64_t{0};
  };

  // the first rows are requested before the partials: the two loads overlap
  RowIn<ROLE> cur;
  cur.load(src, d, group_blk(grp), r);

  // tensor amax: the partials of k_amax_part, or the caller's value
  uint32_t ab;
  if (nparts >= 0) {
    uint32_t m = 0;
    if constexpr (ONE) {
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      const int64_t n4 = d.nblocks * 16;
      int64_t i = threadIdx.x;
      for (; i + 3 * kOneThreads < n4; i += 4 * kOneThreads) {  // 4 loads in flight
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = s4[i + k * kOneThreads];
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max4(v[k]));
      }
      for (; i < n4; i += kOneThreads) m = max(m, max4(s4[i]));
    } else {
      for (int i = lane; i < nparts; i += 64) m = max(m, part[i] & ~kPartTiny);
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
    if constexpr (ONE) {
      __shared__ uint32_t wmax[kOneThreads / 64];
      if (lane == 0) wmax[threadIdx.x >> 6] = m;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kOneThreads / 64; ++k) m = max(m, wmax[k]);
    }
    ab = m;
  } else {
    ab = __float_as_uint(*amax) & 0x7FFFFFFFu;
  }
  const bool nonfinite = ab >= NONFINITE_BITS;
  const float T = nonfinite ? __uint_as_float(0x7FC00000u) : __uint_as_float(ab) / (448.0f * F::MAXV);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *tensor_scale = T;
    if (nparts >= 0) *amax = __uint_as_float(ab);
  }
  const float den = F::MAXV * T;
  const float y_den = 1.0f / den;
  const bool den_ok = (den >= 0x1p-125f) & (den <= 0x1p125f);
  const float thr_den = fmaxf(0x1p-100f, den * 0x1p-98f);

  // two stages: the next group's rows are in flight while this one is coded
  for (; grp < ngroups; grp += gstride) {
    const int64_t blk = grp * 8 + (lane >> 3);
    const bool valid = blk < d.nblocks;
    RowIn<ROLE> nxt;
    nxt.load(src, d, group_blk(grp + gstride), r);
    if (nonfinite) {  // T = NaN, scales 0x7F, codes 0
      store_row<FMT>(codes, blk, r, 0u, 0u, valid);
      if (valid && r == 0) scales[blk] = 0x7F;
      cur = nxt;
      continue;
    }
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) am = fmaxf(fmaxf(am, fabsf(cur.x[j])), fabsf(cur.x[j + 1]));
    am = max8(am);

    // Quotients a / b are computed as RN(a / b) from y = RN(1/b) without a
    // division (div_by_recip); the guards send everything else through the
    // division.  Block scale: the quotient is at most 448 (1 + 2^-23).
    float braw = div_by_recip(am, den, y_den);
    if (!((T == 0.0f) | (den_ok & ((am == 0.0f) | (am >= thr_den))))) braw = am / den;
    braw = (T == 0.0f) ? 0.0f : braw;
    const uint32_t bcode = rne_e4m3_hw(braw);
    const float B = code_value<ScaleFmt>(bcode);
    const float dd = B * T;
    // Elements: |x| / dd is at most 8 * MAXV because dd is the block amax
    // over MAXV rounded to an E4M3 block scale.  A zero block scale gives
    // y = 0, so every quotient is 0 (q = 0, residual a, a * 0 + 0).
    const float y = (dd == 0.0f) ? 0.0f : 1.0f / dd;
    const bool dd_ok = (dd >= 0x1p-125f) & (dd <= 0x1p125f);
    const float thr = fmaxf(0x1p-100f, dd * 0x1p-98f);
    float v[8];
    // a tiny nonzero element, 0 < |x| < thr: 2 bits(|x|) - 1 below
    // 2 bits(thr) - 1 as unsigned (a zero wraps to the maximum)
    uint32_t mn = ~0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = div_by_recip(fabsf(cur.x[j]), dd, y);
      mn = min(mn, (__float_as_uint(cur.x[j]) << 1) - 1u);
    }
    bool any_slow = mn < (__float_as_uint(thr) << 1) - 1u;
    any_slow = (any_slow | !dd_ok) & (dd != 0.0f);
    if (any_slow) {  // rare: tiny elements or an extreme block scale
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ax = fabsf(cur.x[j]);
        if (!dd_ok | ((ax != 0.0f) & (ax < thr))) v[j] = ax / dd;
      }
    }

    uint64_t bits = 0;
    if constexpr (!SR && (FMT == FMT_E2M1 || FMT == FMT_E4M3)) {
      // the hardware conversion rounds to nearest even like rne_code and
      // takes the sign of its input (also of -0); v is clamped to the format
      // maximum first
      float sv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = __builtin_copysignf(fminf(v[j], F::MAXV), cur.x[j]);
      if constexpr (FMT == FMT_E2M1) {
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, sv[0], sv[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, sv[2], sv[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, sv[4], sv[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, sv[6], sv[7], 1.0f, 3);
        bits = w;
      } else {
        short2v lo = {0, 0}, hi = {0, 0};
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, sv[0], sv[1], 1.0f, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, sv[2], sv[3], 1.0f, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, sv[4], sv[5], 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, sv[6], sv[7], 1.0f, true);
        bits = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, lo)) |
               (static_cast<uint64_t>(__builtin_bit_cast(uint32_t, hi)) << 32);
      }
    } else {
      uint32_t ub[8];  // complemented SR uniforms
      if constexpr (SR) {
        if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
          for (int j = 0; j < 8; ++j) ub[j] = sr_ubar(seed, static_cast<uint64_t>(cur.rowbase + j * cur.col));
        } else {
          // a row is 8 consecutive elements from an even index: 4 draws
          uint64_t gk = kGolden64 * (static_cast<uint64_t>(cur.rowbase >> 1) + 1ull);
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            sr_ubar_pair(seed, gk, ub[j], ub[j + 1]);
            gk += kGolden64;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t mag;
        if constexpr (SR) {
          mag = sr_code<F>(v[j], ub[j]);
        } else {
          mag = rne_code<F>(v[j]);
        }
        const uint32_t code = F::SIGNED ? (mag | ((__float_as_uint(cur.x[j]) >> 31) << F::SIGN)) : mag;
        bits |= static_cast<uint64_t>(code) << (F::BITS * j);
      }
    }
    store_row<FMT>(codes, blk, r, static_cast<uint32_t>(bits), static_cast<uint32_t>(bits >> 32), valid);
    if (valid && r == 0) scales[blk] = static_cast<uint8_t>(bcode);
    cur = nxt;
  }
}

// The bulk path for activations and gradients (N contiguous): 32 blocks per
// wave iteration, two lanes per block.  Lane 2b + h holds columns 4h..4h+3
// of the 8 rows of block b, so each of a wave's 8 row loads reads 32
// consecutive 16-byte pieces (1 KiB contiguous when N >= 256, 512-byte runs
// at N = 128), twice the rows in flight of the row-per-lane kernel above.
// After the codes are formed, the lanes of a pair swap half rows so that
// lane h holds whole rows 4h..4h+3 and stores them (half a block) as one
// contiguous run.  The arithmetic per element and per block is that of
// k_quantize, so the codes are identical.
constexpr int kWideBlocks = 32;
template <int FMT, int ROLE, bool SR>
__global__ __launch_bounds__(kThreads) void k_quantize_wide(const float* __restrict__ src,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ tensor_scale,
                                                            float* __restrict__ amax,
                                                            const uint32_t* __restrict__ part, int nparts,
                                                            QDims d, uint64_t seed) {
  static_assert(ROLE != MX_ROLE_WEIGHT, "rows of 8 contiguous elements");
  using F = Fmt<FMT>;
  constexpr int B = F::BITS;
  const int lane = threadIdx.x & 63, h = lane & 1;
  const int64_t ngroups = (d.nblocks + kWideBlocks - 1) / kWideBlocks;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * kGroupsPerWG;
  int64_t grp = static_cast<int64_t>(blockIdx.x) * kGroupsPerWG + (threadIdx.x >> 6);
  const int64_t row = d.d3;  // N
  const uint64_t gk_row = kGolden64 * static_cast<uint64_t>(row >> 1);  // N is a multiple of 8
  struct Rows {
    float4 x[8];  // columns 4h..4h+3 of rows 0..7
    int64_t base;  // source offset of column 4h of row 0
  };
  // launched only for tensors of more than kOneBlocks blocks: block 0 exists
  auto load = [&](Rows& R, int64_t g) {
    int64_t b = g * kWideBlocks + (lane >> 1);
    b = b < d.nblocks ? b : 0;  // past the tensor: block 0, loaded, never stored
    R.base = block_addr<ROLE>(d, b).base + 4 * h;
#pragma unroll
    for (int r = 0; r < 8; ++r) R.x[r] = load_stream(src + R.base + r * row);
  };
  Rows cur;
  load(cur, grp);  // requested before the partials: the two loads overlap

  uint32_t ab;
  bool tiny_free = false;  // no element of the tensor is tiny for any block scale
  if (nparts >= 0) {
    uint32_t m = 0, f = 0;
    for (int i = lane; i < nparts; i += 64) {
      const uint32_t p = part[i];
      m = max(m, p & ~kPartTiny);
      f |= p;
    }
    for (int off = 32; off > 0; off >>= 1) {
      m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
      f |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(f), off));
    }
    ab = m;
    // every nonzero |x| >= 2^-64, and every block's dd <= amax / MAXV <=
    // 2^34, so the bound max(2^-100, dd 2^-98) is at most 2^-64
    tiny_free = __builtin_amdgcn_readfirstlane(((f & kPartTiny) == 0u) & (ab <= 0x50800000u)) != 0;
  } else {
    ab = __float_as_uint(*amax) & 0x7FFFFFFFu;
  }
  const bool nonfinite = ab >= NONFINITE_BITS;
  const float T = nonfinite ? __uint_as_float(0x7FC00000u) : __uint_as_float(ab) / (448.0f * F::MAXV);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *tensor_scale = T;
    if (nparts >= 0) *amax = __uint_as_float(ab);
  }
  const float den = F::MAXV * T;
  const float y_den = 1.0f / den;
  const bool den_ok = (den >= 0x1p-125f) & (den <= 0x1p125f);
  const float thr_den = fmaxf(0x1p-100f, den * 0x1p-98f);
  // Per block-scale code c (0..126): dd = B(c) T, y = RN(1 / dd) (0 where
  // dd = 0, which makes every quotient 0), the tiny-element bound
  // 2 bits(thr) - 1 (0 where dd = 0: nothing is tiny) and 1 where dd is
  // outside the range of the reciprocal quotient (every element divides).
  __shared__ ScaleEntry stab[128];
  if (threadIdx.x < 128) {
    const float dd = code_value<ScaleFmt>(threadIdx.x) * T;
    const bool dd_ok = (dd >= 0x1p-125f) & (dd <= 0x1p125f);
    const float thr = fmaxf(0x1p-100f, dd * 0x1p-98f);
    ScaleEntry e;
    e.dd = dd;
    e.y = (dd == 0.0f) ? 0.0f : 1.0f / dd;
    e.tiny = (dd == 0.0f) ? 0u : (__float_as_uint(thr) << 1) - 1u;
    e.all_slow = (!dd_ok & (dd != 0.0f)) ? 1u : 0u;
    stab[threadIdx.x] = e;
  }
  __syncthreads();
  // the seed in registers before the loop: a wait for its scalar load inside
  // the loop would also wait for the table reads there
  if constexpr (SR) asm volatile("" ::"s"(seed));

  for (; grp < ngroups; grp += gstride) {
    const int64_t blk = grp * kWideBlocks + (lane >> 1);
    const bool valid = blk < d.nblocks;
    Rows nxt;
    load(nxt, grp + gstride);
    uint32_t words[B];  // rows 4h..4h+3 of the block, packed
    uint32_t bcode = 0x7F;  // T = NaN: scales 0x7F, codes 0
#pragma unroll
    for (int k = 0; k < B; ++k) words[k] = 0u;
    if (!nonfinite) {
      // a running chain of maxima (three-operand maxima on the raw loads)
      float am = 0.0f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        am = fmaxf(fmaxf(am, fabsf(cur.x[r].x)), fabsf(cur.x[r].y));
        am = fmaxf(fmaxf(am, fabsf(cur.x[r].z)), fabsf(cur.x[r].w));
      }
      am = fmaxf(am, swap_pair(am));

      float braw = div_by_recip(am, den, y_den);
      const bool braw_div = !((T == 0.0f) | (den_ok & ((am == 0.0f) | (am >= thr_den))));
      if (__builtin_amdgcn_ballot_w64(braw_div)) {  // rare: skipped by the whole wave otherwise
        if (braw_div) braw = am / den;
        asm volatile("" : "+v"(braw));  // keeps the division inside the branch
      }
      braw = (T == 0.0f) ? 0.0f : braw;
      bcode = rne_e4m3_hw(braw);
      const ScaleEntry se = stab[bcode];
      float xs[32], v[32];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        xs[4 * r] = cur.x[r].x; xs[4 * r + 1] = cur.x[r].y;
        xs[4 * r + 2] = cur.x[r].z; xs[4 * r + 3] = cur.x[r].w;
      }
      // a tiny nonzero element, 0 < |x| < thr: 2 bits(|x|) - 1 below
      // 2 bits(thr) - 1 as unsigned (a zero wraps to the maximum), tested
      // on the minimum over the lane's elements (vector operations only),
      // while the table entry is read
      uint32_t mn = ~0u;
      if (!tiny_free) {
#pragma unroll
        for (int j = 0; j < 32; j += 2) mn = min(min(mn, tiny_key(__float_as_uint(xs[j]))), tiny_key(__float_as_uint(xs[j + 1])));
      }
      // SR draws (complemented uniforms) of element 4 r + j: counters of row
      // r of this lane start at element base + r N (even), so its first pair
      // is k0 + r N / 2 with k0 = base / 2 and gk = kGolden64 (k + 1)
      // advances by a constant from row to row (a running 64-bit sum, not a
      // product per row).  Rows 0 and 1 are drawn here, while the table
      // entry is read.
      uint32_t ub[32];
      uint64_t gk = kGolden64 * (static_cast<uint64_t>(cur.base >> 1) + 1ull);
      auto draw_row = [&](int r) {
        sr_ubar_pair(seed, gk, ub[4 * r], ub[4 * r + 1]);
        sr_ubar_pair(seed, gk + kGolden64, ub[4 * r + 2], ub[4 * r + 3]);
        gk += gk_row;
      };
      if constexpr (SR) {
        draw_row(0);
        draw_row(1);
#pragma unroll
        for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(ub[k]));  // drawn here, not at their use
      }
      __builtin_amdgcn_sched_barrier(0);
      const float dd = se.dd, y = se.y;
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = div_by_recip(fabsf(xs[j]), dd, y);
      const bool any_slow = (mn < se.tiny) | (se.all_slow != 0u);
      if (any_slow) {  // rare: tiny elements or an extreme block scale
        const bool dd_ok = se.all_slow == 0u;
        const float thr = fmaxf(0x1p-100f, dd * 0x1p-98f);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float ax = fabsf(xs[j]);
          if (!dd_ok | ((ax != 0.0f) & (ax < thr))) v[j] = ax / dd;
        }
      }

      // the 4 codes of each row of this lane, BITS each
      uint32_t chunk[8];
      if constexpr (!SR && (FMT == FMT_E2M1 || FMT == FMT_E4M3)) {
        // hardware round to nearest even on copysign(min(v, max), x)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          float sv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) sv[j] = __builtin_copysignf(fminf(v[4 * r + j], F::MAXV), xs[4 * r + j]);
          if constexpr (FMT == FMT_E2M1) {
            uint32_t w = 0;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, sv[0], sv[1], 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, sv[2], sv[3], 1.0f, 1);
            chunk[r] = w & 0xFFFFu;
          } else {
            short2v c = {0, 0};
            c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, sv[0], sv[1], 1.0f, false);
            c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, sv[2], sv[3], 1.0f, true);
            chunk[r] = __builtin_bit_cast(uint32_t, c);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if constexpr (SR) {
            if (r >= 2) draw_row(r);
          }
          uint32_t c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t mag;
            if constexpr (SR) mag = sr_code<F>(v[4 * r + j], ub[4 * r + j]);
            else mag = rne_code<F>(v[4 * r + j]);
            const uint32_t code = F::SIGNED ? (mag | ((__float_as_uint(xs[4 * r + j]) >> 31) << F::SIGN)) : mag;
            c |= code << (B * j);
          }
          chunk[r] = c;
        }
      }

      // pair exchange: lane 0 of the pair keeps rows 0..3 and takes their
      // columns 4..7 from lane 1, which keeps rows 4..7 and takes their
      // columns 0..3
      uint64_t rows4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t recv = swap_pair(h ? chunk[r] : chunk[r + 4]);
        const uint32_t lo = h ? recv : chunk[r];
        const uint32_t hi = h ? chunk[r + 4] : recv;
        rows4[r] = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << (4 * B));
      }
      // 4 rows of 8 B bits, little-endian, into B words.  The bits still
      // pending when a row is added (0 for B = 4 and 8, 0 or 16 for B = 6,
      // 0, 8, 16 or 24 for B = 3) plus the row never exceed 64.
      static_assert(B == 3 || B == 4 || B == 6 || B == 8, "code widths of the formats");
      uint64_t acc = 0;
      int nb = 0, nw = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc |= rows4[r] << nb;
        nb += 8 * B;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (nb >= 32) {
            words[nw++] = static_cast<uint32_t>(acc);
            acc >>= 32;
            nb -= 32;
          }
        }
      }
    }
    if (valid) {
      uint8_t* q = codes + blk * (8 * B) + h * (4 * B);
      if constexpr (B == 4) {
        *reinterpret_cast<uint4*>(q) = make_uint4(words[0], words[1], words[2], words[3]);
      } else if constexpr (B == 8) {
        reinterpret_cast<uint4*>(q)[0] = make_uint4(words[0], words[1], words[2], words[3]);
        reinterpret_cast<uint4*>(q)[1] = make_uint4(words[4], words[5], words[6], words[7]);
      } else if constexpr (B == 6) {
#pragma unroll
        for (int k = 0; k < 3; ++k) reinterpret_cast<uint2*>(q)[k] = make_uint2(words[2 * k], words[2 * k + 1]);
      } else {
#pragma unroll
        for (int k = 0; k < B; ++k) reinterpret_cast<uint32_t*>(q)[k] = words[k];
      }
      if (h == 0) scales[blk] = static_cast<uint8_t>(bcode);
    }
    cur = nxt;
  }
}

// One code row of a block as a 64-bit value (8 codes, BITS each).
template <int FMT>
__device__ __forceinline__ uint64_t load_row(const uint8_t* __restrict__ codes, int64_t blk, int r) {
  if constexpr (FMT == FMT_E2M1) {
    return *reinterpret_cast<const uint32_t*>(codes + blk * 32 + r * 4);
  } else if constexpr (FMT == FMT_E4M3) {
    const uint2 v = *reinterpret_cast<const uint2*>(codes + blk * 64 + r * 8);
    return static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32);
  } else if constexpr (FMT == FMT_UE2M1) {
    // bytes 3r .. 3r+2 of the 24-byte block: in word 3r/4 and the next one,
    // except for row 7, whose bytes all lie in word 5 (the last of the block)
    const int off = 3 * r;
    const uint32_t* q = reinterpret_cast<const uint32_t*>(codes + blk * 24);
    const int w0 = off >> 2, w1 = w0 + 1 < 6 ? w0 + 1 : 5;
    const uint64_t v = static_cast<uint64_t>(q[w0]) | (static_cast<uint64_t>(q[w1]) << 32);
    return (v >> ((off & 3) * 8)) & 0xFFFFFFull;
  } else {
    // bytes 6r .. 6r+5 lie inside the two dwords starting at floor(6r/4)
    const int off = 6 * r;
    const uint32_t* q = reinterpret_cast<const uint32_t*>(codes + blk * 48) + (off >> 2);
    const uint64_t v = static_cast<uint64_t>(q[0]) | (static_cast<uint64_t>(q[1]) << 32);
    return (v >> ((off & 3) * 8)) & 0xFFFFFFFFFFFFull;
  }
}

// 8 lanes per block, lane = block row, as in k_quantize.
template <int FMT, int ROLE>
__global__ __launch_bounds__(kThreads) void k_dequantize(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ tensor_scale,
                                                         float* __restrict__ dst, QDims d) {
  using F = Fmt<FMT>;
  const int r = threadIdx.x & 7;
  const int64_t blk = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 3;
  if (blk >= d.nblocks) return;
  const uint64_t row = load_row<FMT>(codes, blk, r);
  const uint32_t sb = scales[blk];
  const float B = (sb == 0x7Fu) ? __uint_as_float(0x7FC00000u) : code_value<ScaleFmt>(sb);
  const float T = *tensor_scale;
  const BlockAddr ad = block_addr<ROLE>(d, blk);
  const int64_t rowbase = ad.base + r * ad.row;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t code = static_cast<uint32_t>(row >> (F::BITS * j)) & ((1u << F::BITS) - 1u);
    const float g = code_value<F>(code & ((1u << F::SIGN) - 1u));
    const float gb = g * B;
    float v = gb * T;
    if (F::SIGNED && ((code >> F::SIGN) & 1u)) v = -v;
    o[j] = v;
  }
  if constexpr (ROLE == MX_ROLE_WEIGHT) {
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[rowbase + j * ad.col] = o[j];
  } else {
    *reinterpret_cast<float4*>(dst + rowbase) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dst + rowbase + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// Activations and gradients, the layout of k_quantize_wide: two lanes per
// block, lane 2b + h writing columns 4h..4h+3 of the 8 rows of block b, so
// that each of a wave's 8 row stores covers 32 consecutive 16-byte pieces
// (1 KiB contiguous when N >= 256).  Both lanes of a pair read the whole
// block of codes (the same 64-byte segment).  Values as in k_dequantize.
template <int FMT, int ROLE, bool STREAM>
__global__ __launch_bounds__(kThreads) void k_dequantize_wide(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ tensor_scale,
                                                              float* __restrict__ dst, QDims d) {
  static_assert(ROLE != MX_ROLE_WEIGHT, "rows of 8 contiguous elements");
  using F = Fmt<FMT>;
  constexpr int B = F::BITS;
  constexpr int NW = 2 * B;  // 32-bit words of a block (8 rows of 8 B bits)
  const int h = threadIdx.x & 1;
  const int64_t blk = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 1;
  if (blk >= d.nblocks) return;
  uint32_t w[NW];
  const uint8_t* q = codes + blk * (8 * B);
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int k = 0; k < NW / 4; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(q)[k];
      w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
  } else if constexpr (NW % 2 == 0 && (8 * B) % 8 == 0) {
#pragma unroll
    for (int k = 0; k < NW / 2; ++k) {
      const uint2 v = reinterpret_cast<const uint2*>(q)[k];
      w[2 * k] = v.x; w[2 * k + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = reinterpret_cast<const uint32_t*>(q)[k];
  }
  // 4B bits at a compile-time bit offset o of the block
  auto field = [&](int o) -> uint32_t {
    const int k = o >> 5, sh = o & 31;
    const uint64_t v = static_cast<uint64_t>(w[k]) | (k + 1 < NW ? static_cast<uint64_t>(w[k + 1]) << 32 : 0ull);
    return static_cast<uint32_t>(v >> sh) & static_cast<uint32_t>((1ull << (4 * B)) - 1ull);
  };
  const uint32_t sb = scales[blk];
  const float Bv = (sb == 0x7Fu) ? __uint_as_float(0x7FC00000u) : code_value<ScaleFmt>(sb);
  const float T = *tensor_scale;
  const int64_t base = block_addr<ROLE>(d, blk).base + 4 * h;
  const int64_t row = d.d3;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t f = h ? field(8 * B * r + 4 * B) : field(8 * B * r);
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t code = (f >> (B * j)) & ((1u << B) - 1u);
      const float g = code_value<F>(code & ((1u << F::SIGN) - 1u));
      const float gb = g * Bv;
      float v = gb * T;
      if (F::SIGNED && ((code >> F::SIGN) & 1u)) v = -v;
      o[j] = v;
    }
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const f32x4v ov = {o[0], o[1], o[2], o[3]};
    f32x4v* q = reinterpret_cast<f32x4v*>(dst + base + r * row);
    if constexpr (STREAM) __builtin_nontemporal_store(ov, q);  // outputs above kStreamOutBytes
    else *q = ov;
  }
}

// Explicit channel-batch-first im2col, the baseline the paper compares
// against (quantize after im2col, §III-C): X' [Ho][Wo][Kh][Kw][C][N] from X
// [H][W][C][N], zero where a tap falls in the padding.  Each (ho, wo, kh, kw)
// row is C*N contiguous floats of X at one position, copied with 16-byte
// loads and stores; a workgroup copies whole rows.
__global__ __launch_bounds__(256) void k_im2col_cbf(const float4* __restrict__ x, float4* __restrict__ xc,
                                                    int h, int w, int k_h, int k_w, int sh, int sw, int ph,
                                                    int pw, int wo, int64_t row4, int64_t rows) {
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    int64_t t = row;
    const int kw = static_cast<int>(t % k_w); t /= k_w;
    const int kh = static_cast<int>(t % k_h); t /= k_h;
    const int ox = static_cast<int>(t % wo);
    const int oy = static_cast<int>(t / wo);
    const int iy = oy * sh - ph + kh, ix = ox * sw - pw + kw;
    const bool in = iy >= 0 && iy < h && ix >= 0 && ix < w;
    float4* dst = xc + row * row4;
    if (in) {
      const float4* src = x + (static_cast<int64_t>(iy) * w + ix) * row4;
      for (int64_t i = threadIdx.x; i < row4; i += 256) dst[i] = src[i];
    } else {
      for (int64_t i = threadIdx.x; i < row4; i += 256) dst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
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
  d.m_nb = d.m_cb = 0;
  d.s_nb = d.s_cb = 0;
  if (role != MX_ROLE_WEIGHT) {
    magic_div(static_cast<uint32_t>(d.d3 >> 3), d.m_nb, d.s_nb);
    magic_div(static_cast<uint32_t>(d.d2 >> 3), d.m_cb, d.s_cb);
  }
  return d;
}

template <int FMT, int ROLE>
void launch_q(const QDims& d, const float* src, const mx_qtensor* q, bool sr, uint64_t seed,
              const uint32_t* part, int nparts, bool one, hipStream_t s) {
  auto* codes = static_cast<uint8_t*>(q->codes);
  if (one) {  // nparts >= 0: the kernel computes the amax itself
    if (sr)
      hipLaunchKernelGGL((k_quantize<FMT, ROLE, true, true>), dim3(1), dim3(kOneThreads), 0, s, src, codes,
                         q->scales, q->tensor_scale, q->amax, part, nparts, d, seed);
    else
      hipLaunchKernelGGL((k_quantize<FMT, ROLE, false, true>), dim3(1), dim3(kOneThreads), 0, s, src, codes,
                         q->scales, q->tensor_scale, q->amax, part, nparts, d, seed);
    return;
  }
  if constexpr (ROLE != MX_ROLE_WEIGHT) {
    // at least one workgroup, so that an empty tensor still publishes T
    int64_t wgs = (d.nblocks + kWideBlocks * kGroupsPerWG - 1) / (kWideBlocks * kGroupsPerWG);
    if (wgs > kQuantMaxWGs) wgs = kQuantMaxWGs;
    if (wgs < 1) wgs = 1;
    const dim3 grid(static_cast<unsigned>(wgs));
    if (sr)
      hipLaunchKernelGGL((k_quantize_wide<FMT, ROLE, true>), grid, dim3(kThreads), 0, s, src, codes, q->scales,
                         q->tensor_scale, q->amax, part, nparts, d, seed);
    else
      hipLaunchKernelGGL((k_quantize_wide<FMT, ROLE, false>), grid, dim3(kThreads), 0, s, src, codes, q->scales,
                         q->tensor_scale, q->amax, part, nparts, d, seed);
  } else {
    // weights: one lane per block row (the rows are strided gathers)
    int64_t wgs = (d.nblocks + 8 * kGroupsPerWG - 1) / (8 * kGroupsPerWG);
    if (wgs > kQuantMaxWGs) wgs = kQuantMaxWGs;
    if (wgs < 1) wgs = 1;
    const dim3 grid(static_cast<unsigned>(wgs));
    if (sr)
      hipLaunchKernelGGL((k_quantize<FMT, ROLE, true, false>), grid, dim3(kThreads), 0, s, src, codes, q->scales,
                         q->tensor_scale, q->amax, part, nparts, d, seed);
    else
      hipLaunchKernelGGL((k_quantize<FMT, ROLE, false, false>), grid, dim3(kThreads), 0, s, src, codes, q->scales,
                         q->tensor_scale, q->amax, part, nparts, d, seed);
  }
}

template <int FMT>
void launch_q_role(mx_role role, const QDims& d, const float* src, const mx_qtensor* q, bool sr,
                   uint64_t seed, const uint32_t* part, int nparts, bool one, hipStream_t s) {
  if (role == MX_ROLE_ACT) launch_q<FMT, MX_ROLE_ACT>(d, src, q, sr, seed, part, nparts, one, s);
  else if (role == MX_ROLE_GRAD) launch_q<FMT, MX_ROLE_GRAD>(d, src, q, sr, seed, part, nparts, one, s);
  else launch_q<FMT, MX_ROLE_WEIGHT>(d, src, q, sr, seed, part, nparts, one, s);
}

template <int FMT, int ROLE>
void launch_dq(const QDims& d, const mx_qtensor* q, float* dst, hipStream_t s) {
  if constexpr (ROLE != MX_ROLE_WEIGHT) {
    const int64_t wgs = (d.nblocks * 2 + kThreads - 1) / kThreads;
    if (wgs == 0) return;
    const auto* codes = static_cast<const uint8_t*>(q->codes);
    if (static_cast<size_t>(d.nblocks) * 64 * sizeof(float) > kStreamOutBytes)
      hipLaunchKernelGGL((k_dequantize_wide<FMT, ROLE, true>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
                         codes, q->scales, q->tensor_scale, dst, d);
    else
      hipLaunchKernelGGL((k_dequantize_wide<FMT, ROLE, false>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
                         codes, q->scales, q->tensor_scale, dst, d);
    return;
  }
  const int64_t wgs = (d.nblocks * 8 + kThreads - 1) / kThreads;
  if (wgs == 0) return;
  hipLaunchKernelGGL((k_dequantize<FMT, ROLE>), dim3(static_cast<unsigned>(wgs)), dim3(kThreads), 0, s,
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
  const bool sr = rounding == MX_SR;
  // small tensors: one workgroup, amax included; otherwise the partials of
  // the amax pass go into the scales buffer, behind the block scales
  const bool one = d.nblocks <= kOneBlocks;
  uint32_t* part = nullptr;
  int nparts = amax_given ? -1 : 0;  // -1: the caller's amax
  if (!amax_given && !one) {
    const int64_t n4 = d.nblocks * 16;
    nparts = static_cast<int>(amax_partials(d.nblocks));
    if (nparts > 0) {
      part = reinterpret_cast<uint32_t*>(dst->scales + scale_tail_offset(d.nblocks));
      hipLaunchKernelGGL(k_amax_part, dim3(static_cast<unsigned>(nparts)), dim3(kAmaxThreads), 0, s,
                         reinterpret_cast<const uint4*>(src), n4, part);
    }
  }
  switch (role_fmt(g, role)) {
    case FMT_E2M1: launch_q_role<FMT_E2M1>(role, d, src, dst, sr, seed, part, nparts, one, s); break;
    case FMT_E2M3: launch_q_role<FMT_E2M3>(role, d, src, dst, sr, seed, part, nparts, one, s); break;
    case FMT_E3M2: launch_q_role<FMT_E3M2>(role, d, src, dst, sr, seed, part, nparts, one, s); break;
    case FMT_UE2M1: launch_q<FMT_UE2M1, MX_ROLE_ACT>(d, src, dst, sr, seed, part, nparts, one, s); break;
    default: launch_q_role<FMT_E4M3>(role, d, src, dst, sr, seed, part, nparts, one, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_im2col(const Geom& g, const float* x, float* xcol, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(g.ho) * g.wo * g.k_h * g.k_w;
  const int64_t row4 = static_cast<int64_t>(g.c_in) * g.n / 4;  // C*N is a multiple of 64
  if (rows == 0 || row4 == 0) return hipSuccess;
  const unsigned wgs = static_cast<unsigned>(rows < 65536 ? rows : 65536);
  hipLaunchKernelGGL(k_im2col_cbf, dim3(wgs), dim3(256), 0, s, reinterpret_cast<const float4*>(x),
                     reinterpret_cast<float4*>(xcol), g.h, g.w, g.k_h, g.k_w, g.sh, g.sw, g.ph, g.pw, g.wo,
                     row4, rows);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Geom& g, mx_role role, const mx_qtensor* q, float* dst,
                             hipStream_t s) {
  const QDims d = make_qdims(g, role);
  switch (role_fmt(g, role)) {
    case FMT_E2M1: launch_dq_role<FMT_E2M1>(role, d, q, dst, s); break;
    case FMT_E2M3: launch_dq_role<FMT_E2M3>(role, d, q, dst, s); break;
    case FMT_E3M2: launch_dq_role<FMT_E3M2>(role, d, q, dst, s); break;
    case FMT_UE2M1: launch_dq<FMT_UE2M1, MX_ROLE_ACT>(d, q, dst, s); break;
    default: launch_dq_role<FMT_E4M3>(role, d, q, dst, s); break;
  }
  return hipGetLastError();
}

}  // namespace mx
