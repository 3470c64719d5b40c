// Internal interface between the C ABI (capi.cpp) and the HIP kernels.
// Arguments reaching these launchers have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxconv.h"

namespace mx {

// Geometry shared by all launchers, derived from an mx_conv_desc.
// fmt: element format of weights and output gradients; afmt: that of the
// activation (the descriptor's act_fmt, or fmt where that is 0).
// block: 8 (the two-level E4M3 x fp32 format) or 32 (E8M0 per 32x32 block).
struct Geom {
  int32_t n, c_in, c_out, h, w, k_h, k_w, sh, sw, ph, pw, ho, wo, fmt, afmt, block;
};
inline int role_fmt(const Geom& g, mx_role role) { return role == MX_ROLE_ACT ? g.afmt : g.fmt; }

Geom make_geom(const mx_conv_desc* d);

// fp32 element count and 8x8 block count of the tensor of `role`.
int64_t role_numel(const Geom& g, mx_role role);
int64_t role_nblocks(const Geom& g, mx_role role);
int code_bits(int fmt);

// fp32 outputs larger than this (the 256 MB last-level cache of the GPU)
// are written with nontemporal stores: they stream past the cache, which
// cannot hold them for a consumer anyway.  Smaller outputs stay cacheable.
constexpr size_t kStreamOutBytes = size_t{256} << 20;

// The scales buffer of a quantized tensor holds the block scales (one byte
// per block), padded to 16 bytes, then the quantizer's amax partials: one
// 32-bit max per workgroup of the amax pass, at most kAmaxMaxPartials.
constexpr int kAmaxMaxPartials = 512;
inline int64_t scale_tail_offset(int64_t nblocks) { return (nblocks + 15) & ~static_cast<int64_t>(15); }
inline int64_t amax_partials(int64_t nblocks) {
  if (nblocks <= 0) return 0;
  const int64_t p = (nblocks * 16 + 4095) / 4096;  // >= 4096 uint4 loads per workgroup
  return p < kAmaxMaxPartials ? p : kAmaxMaxPartials;
}
inline int64_t scale_buffer_bytes(int64_t nblocks) {
  return nblocks > 0 ? scale_tail_offset(nblocks) + 4 * kAmaxMaxPartials : 0;
}
// E8M0 32x32 blocks: the scales alone (no amax pass, no scratch tail).
inline int64_t mx_scale_buffer_bytes(int64_t nblocks) { return nblocks > 0 ? scale_tail_offset(nblocks) : 0; }

hipError_t launch_quantize(const Geom& g, mx_role role, const float* src, const mx_qtensor* dst,
                           mx_round rounding, uint64_t seed, int amax_given, hipStream_t s);
hipError_t launch_dequantize(const Geom& g, mx_role role, const mx_qtensor* q, float* dst,
                             hipStream_t s);
// The E8M0 32x32-block format (quantize_mx.hip).
hipError_t launch_quantize_mx(const Geom& g, mx_role role, const float* src, const mx_qtensor* dst,
                              mx_round rounding, uint64_t seed, hipStream_t s);
hipError_t launch_dequantize_mx(const Geom& g, mx_role role, const mx_qtensor* q, float* dst, hipStream_t s);
hipError_t launch_im2col(const Geom& g, const float* x, float* xcol, hipStream_t s);

// y_amax: nullptr, or a device buffer of fwd_amax_bytes(g) bytes whose first
// word receives max |y| (exact); the rest holds the per-wave partial maxima
hipError_t launch_conv_fwd(const Geom& g, const mx_qtensor* wq, const mx_qtensor* xq, float* y,
                           float* y_amax, hipStream_t s);
size_t fwd_amax_bytes(const Geom& g);
hipError_t launch_conv_dgrad(const Geom& g, const mx_qtensor* wq, const mx_qtensor* dyq, float* dx,
                             hipStream_t s);
hipError_t launch_conv_wgrad(const Geom& g, const mx_qtensor* dyq, const mx_qtensor* xq, float* dw,
                             void* workspace, hipStream_t s);
size_t wgrad_workspace_bytes(const Geom& g);

}  // namespace mx
