// C ABI of the MicroQonv hot path: host-side validation and dispatch.
//
// Every check below runs on the host before anything is enqueued, so the
// error paths need no GPU.  The layouts and the meaning of each argument are
// documented in include/mxconv.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <limits>
#include <mutex>

#include "internal.h"

namespace mx {

Geom make_geom(const mx_conv_desc* d) {
  Geom g;
  g.n = d->n; g.c_in = d->c_in; g.c_out = d->c_out; g.h = d->h; g.w = d->w;
  g.k_h = d->k_h; g.k_w = d->k_w; g.sh = d->stride_h; g.sw = d->stride_w;
  g.ph = d->pad_h; g.pw = d->pad_w; g.fmt = d->elem_fmt;
  g.afmt = d->act_fmt != 0 ? d->act_fmt : d->elem_fmt;
  g.block = d->block;
  g.ho = (d->h + 2 * d->pad_h - d->k_h) / d->stride_h + 1;
  g.wo = (d->w + 2 * d->pad_w - d->k_w) / d->stride_w + 1;
  return g;
}

int64_t role_numel(const Geom& g, mx_role role) {
  switch (role) {
    case MX_ROLE_ACT: return static_cast<int64_t>(g.h) * g.w * g.c_in * g.n;
    case MX_ROLE_GRAD: return static_cast<int64_t>(g.ho) * g.wo * g.c_out * g.n;
    default: return static_cast<int64_t>(g.c_out) * g.c_in * g.k_h * g.k_w;
  }
}

int64_t role_nblocks(const Geom& g, mx_role role) {
  return role_numel(g, role) / (static_cast<int64_t>(g.block) * g.block);
}

int code_bits(int fmt) {
  return fmt == MX_E2M1 ? 4 : (fmt == MX_E2M3 || fmt == MX_E3M2) ? 6 : fmt == MX_UE2M1 ? 3 : 8;
}

}  // namespace mx

namespace {

using mx::Geom;

// Largest element count any one tensor may have (block indices are 32-bit
// inside the conv kernels: 2^31 blocks of 64 elements).
constexpr int64_t kMaxElems = (static_cast<int64_t>(1) << 31) * 64 - 64;
// Geometry products fed to 32-bit kernel arithmetic must stay below this.
constexpr int64_t kMaxIndex = std::numeric_limits<int32_t>::max();

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool known_fmt(int32_t f) {
  return f == MX_E2M1 || f == MX_E2M3 || f == MX_E4M3 || f == MX_UE2M1 || f == MX_E3M2;
}

mx_status check_desc(const mx_conv_desc* d) {
  if (!d) return MX_ERR_NULL;
  if (d->block != 8 && d->block != 32) return MX_ERR_BLOCK;
  if (!known_fmt(d->elem_fmt) || (d->act_fmt != 0 && !known_fmt(d->act_fmt))) return MX_ERR_FORMAT;
  if (d->n < 0 || d->c_in <= 0 || d->c_out <= 0 || d->h <= 0 || d->w <= 0 || d->k_h <= 0 || d->k_w <= 0)
    return MX_ERR_SHAPE;
  if (d->stride_h <= 0 || d->stride_w <= 0 || d->pad_h < 0 || d->pad_w < 0) return MX_ERR_SHAPE;
  if (d->n % d->block || d->c_in % d->block || d->c_out % d->block) return MX_ERR_SHAPE;
  // the E8M0 32x32-block format is implemented for E2M1 elements throughout
  if (d->block == 32 && (d->elem_fmt != MX_E2M1 || (d->act_fmt != 0 && d->act_fmt != MX_E2M1)))
    return MX_ERR_FORMAT;
  if (static_cast<int64_t>(d->h) + 2 * static_cast<int64_t>(d->pad_h) < d->k_h) return MX_ERR_SHAPE;
  if (static_cast<int64_t>(d->w) + 2 * static_cast<int64_t>(d->pad_w) < d->k_w) return MX_ERR_SHAPE;
  const Geom g = mx::make_geom(d);
  if (g.ho <= 0 || g.wo <= 0) return MX_ERR_SHAPE;
  const int64_t nx = mx::role_numel(g, MX_ROLE_ACT), ny = mx::role_numel(g, MX_ROLE_GRAD),
                nw = mx::role_numel(g, MX_ROLE_WEIGHT);
  if (nx > kMaxElems || ny > kMaxElems || nw > kMaxElems) return MX_ERR_SHAPE;
  // column-block and k-block counts of the three GEMMs are 32-bit
  const int64_t kkc = static_cast<int64_t>(d->k_h) * d->k_w * d->c_in;
  if (static_cast<int64_t>(g.h) * g.w * (d->n / 8) > kMaxIndex ||
      static_cast<int64_t>(g.ho) * g.wo * (d->n / 8) > kMaxIndex || kkc > kMaxIndex ||
      static_cast<int64_t>(d->c_out) * kkc > kMaxIndex)
    return MX_ERR_SHAPE;
  return MX_OK;
}

// The compact 3-bit activation codes are a storage format (the replay
// buffer): activations only, and no GEMM reads them.
mx_status check_role_fmt(const mx_conv_desc* d, mx_role role) {
  return (mx::role_fmt(mx::make_geom(d), role) == MX_UE2M1 && role != MX_ROLE_ACT) ? MX_ERR_FORMAT : MX_OK;
}

// Operand formats a GEMM takes: one format for both operands, or E2M1 with
// an FP6 activation (MicroQonv+).  The data gradient reads no activation.
enum class Gemm { Fwd, Dgrad, Wgrad };
mx_status check_gemm_desc(const mx_conv_desc* d, Gemm op) {
  const mx_status st = check_desc(d);
  if (st != MX_OK) return st;
  const Geom g = mx::make_geom(d);
  const int fa = g.fmt, fb = op == Gemm::Dgrad ? g.fmt : g.afmt;
  if (fa == MX_UE2M1 || fb == MX_UE2M1) return MX_ERR_FORMAT;
  if (fa == fb || (fa == MX_E2M1 && (fb == MX_E2M3 || fb == MX_E3M2))) return MX_OK;
  return MX_ERR_FORMAT;
}


mx_status check_role(mx_role r) {
  return (r == MX_ROLE_ACT || r == MX_ROLE_WEIGHT || r == MX_ROLE_GRAD) ? MX_OK : MX_ERR_ROLE;
}

mx_status check_qtensor(const mx_qtensor* q, int64_t nblocks) {
  if (!q) return MX_ERR_NULL;
  if (!q->tensor_scale || !q->amax) return MX_ERR_NULL;
  if (nblocks > 0 && (!q->codes || !q->scales)) return MX_ERR_NULL;
  if (!aligned(q->codes, 16) || !aligned(q->tensor_scale, 4) || !aligned(q->amax, 4)) return MX_ERR_ALIGN;
  return MX_OK;
}

mx_status launched(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH; }

// Weight-gradient workspace of mx_conv_wgrad_noalloc: a static array in
// device memory, one copy per GPU, held until the process ends.  Host code
// never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and cached here.
static __device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, nullptr until looked up

// Device address of the current device's `scratch`.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t mx_code_bytes(const mx_conv_desc* desc, mx_role role) {
  if (check_desc(desc) != MX_OK || check_role(role) != MX_OK) return 0;
  const Geom g = mx::make_geom(desc);
  return static_cast<size_t>(mx::role_numel(g, role)) * mx::code_bits(mx::role_fmt(g, role)) / 8;
}

size_t mx_scale_bytes(const mx_conv_desc* desc, mx_role role) {
  if (check_desc(desc) != MX_OK || check_role(role) != MX_OK) return 0;
  const int64_t nb = mx::role_nblocks(mx::make_geom(desc), role);
  return static_cast<size_t>(desc->block == 32 ? mx::mx_scale_buffer_bytes(nb) : mx::scale_buffer_bytes(nb));
}

size_t mx_wgrad_workspace_bytes(const mx_conv_desc* desc) {
  if (check_gemm_desc(desc, Gemm::Wgrad) != MX_OK) return 0;
  return mx::wgrad_workspace_bytes(mx::make_geom(desc));
}

mx_status mx_quantize_cbf(const mx_conv_desc* desc, mx_role role, const float* src,
                          const mx_qtensor* dst, mx_round rounding, uint64_t seed, int amax_given,
                          hipStream_t stream) {
  mx_status st = check_desc(desc);
  if (st != MX_OK) return st;
  if ((st = check_role(role)) != MX_OK) return st;
  if ((st = check_role_fmt(desc, role)) != MX_OK) return st;
  if (rounding != MX_RNE && rounding != MX_SR) return MX_ERR_ROUND;
  const Geom g = mx::make_geom(desc);
  const int64_t nb = mx::role_nblocks(g, role);
  if ((st = check_qtensor(dst, nb)) != MX_OK) return st;
  if (nb > 0 && !src) return MX_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst->scales, 16)) return MX_ERR_ALIGN;
  if (g.block == 32) return launched(mx::launch_quantize_mx(g, role, src, dst, rounding, seed, stream));
  return launched(mx::launch_quantize(g, role, src, dst, rounding, seed, amax_given, stream));
}

mx_status mx_dequantize(const mx_conv_desc* desc, mx_role role, const mx_qtensor* q, float* dst,
                        hipStream_t stream) {
  mx_status st = check_desc(desc);
  if (st != MX_OK) return st;
  if ((st = check_role(role)) != MX_OK) return st;
  if ((st = check_role_fmt(desc, role)) != MX_OK) return st;
  const Geom g = mx::make_geom(desc);
  const int64_t nb = mx::role_nblocks(g, role);
  if ((st = check_qtensor(q, nb)) != MX_OK) return st;
  if (nb > 0 && !dst) return MX_ERR_NULL;
  if (!aligned(dst, 16)) return MX_ERR_ALIGN;
  if (g.block == 32) return launched(mx::launch_dequantize_mx(g, role, q, dst, stream));
  return launched(mx::launch_dequantize(g, role, q, dst, stream));
}

mx_status mx_conv_fwd(const mx_conv_desc* desc, const mx_qtensor* wq, const mx_qtensor* xq, float* y,
                      hipStream_t stream) {
  mx_status st = check_gemm_desc(desc, Gemm::Fwd);
  if (st != MX_OK) return st;
  const Geom g = mx::make_geom(desc);
  if ((st = check_qtensor(wq, mx::role_nblocks(g, MX_ROLE_WEIGHT))) != MX_OK) return st;
  if ((st = check_qtensor(xq, mx::role_nblocks(g, MX_ROLE_ACT))) != MX_OK) return st;
  if (mx::role_numel(g, MX_ROLE_GRAD) > 0 && !y) return MX_ERR_NULL;
  if (!aligned(y, 16)) return MX_ERR_ALIGN;
  return launched(mx::launch_conv_fwd(g, wq, xq, y, nullptr, stream));
}

mx_status mx_im2col_cbf(const mx_conv_desc* desc, const float* x, float* xcol, hipStream_t stream) {
  mx_status st = check_desc(desc);
  if (st != MX_OK) return st;
  const Geom g = mx::make_geom(desc);
  const int64_t nx = mx::role_numel(g, MX_ROLE_ACT);
  const int64_t nc = static_cast<int64_t>(g.ho) * g.wo * g.k_h * g.k_w * g.c_in * g.n;
  if ((nx > 0 && !x) || (nc > 0 && !xcol)) return MX_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xcol, 16)) return MX_ERR_ALIGN;
  return launched(mx::launch_im2col(g, x, xcol, stream));
}

size_t mx_fwd_amax_bytes(const mx_conv_desc* desc) {
  if (check_gemm_desc(desc, Gemm::Fwd) != MX_OK || desc->block != 8) return 0;
  return mx::fwd_amax_bytes(mx::make_geom(desc));
}

mx_status mx_conv_fwd_amax(const mx_conv_desc* desc, const mx_qtensor* wq, const mx_qtensor* xq, float* y,
                           float* y_amax, hipStream_t stream) {
  mx_status st = check_gemm_desc(desc, Gemm::Fwd);
  if (st != MX_OK) return st;
  // a tensor amax feeds the two-level format only
  if (desc->block != 8) return MX_ERR_BLOCK;
  const Geom g = mx::make_geom(desc);
  if ((st = check_qtensor(wq, mx::role_nblocks(g, MX_ROLE_WEIGHT))) != MX_OK) return st;
  if ((st = check_qtensor(xq, mx::role_nblocks(g, MX_ROLE_ACT))) != MX_OK) return st;
  if (mx::role_numel(g, MX_ROLE_GRAD) > 0 && !y) return MX_ERR_NULL;
  if (!y_amax) return MX_ERR_NULL;
  if (!aligned(y, 16) || !aligned(y_amax, 4)) return MX_ERR_ALIGN;
  return launched(mx::launch_conv_fwd(g, wq, xq, y, y_amax, stream));
}

mx_status mx_conv_dgrad(const mx_conv_desc* desc, const mx_qtensor* wq, const mx_qtensor* dyq,
                        float* dx, hipStream_t stream) {
  mx_status st = check_gemm_desc(desc, Gemm::Dgrad);
  if (st != MX_OK) return st;
  const Geom g = mx::make_geom(desc);
  if ((st = check_qtensor(wq, mx::role_nblocks(g, MX_ROLE_WEIGHT))) != MX_OK) return st;
  if ((st = check_qtensor(dyq, mx::role_nblocks(g, MX_ROLE_GRAD))) != MX_OK) return st;
  if (mx::role_numel(g, MX_ROLE_ACT) > 0 && !dx) return MX_ERR_NULL;
  if (!aligned(dx, 16)) return MX_ERR_ALIGN;
  return launched(mx::launch_conv_dgrad(g, wq, dyq, dx, stream));
}

mx_status mx_conv_wgrad(const mx_conv_desc* desc, const mx_qtensor* dyq, const mx_qtensor* xq,
                        float* dw, void* workspace, size_t ws_bytes, hipStream_t stream) {
  mx_status st = check_gemm_desc(desc, Gemm::Wgrad);
  if (st != MX_OK) return st;
  const Geom g = mx::make_geom(desc);
  if ((st = check_qtensor(dyq, mx::role_nblocks(g, MX_ROLE_GRAD))) != MX_OK) return st;
  if ((st = check_qtensor(xq, mx::role_nblocks(g, MX_ROLE_ACT))) != MX_OK) return st;
  if (!dw) return MX_ERR_NULL;
  if (!aligned(dw, 16)) return MX_ERR_ALIGN;
  const size_t need = mx::wgrad_workspace_bytes(g);
  if (need > 0 && (!workspace || ws_bytes < need)) return MX_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return MX_ERR_ALIGN;
  return launched(mx::launch_conv_wgrad(g, dyq, xq, dw, workspace, stream));
}

mx_status mx_conv_wgrad_noalloc(const mx_conv_desc* desc, const mx_qtensor* dyq, const mx_qtensor* xq,
                                float* dw, hipStream_t stream) {
  mx_status st = check_gemm_desc(desc, Gemm::Wgrad);
  if (st != MX_OK) return st;
  const Geom g = mx::make_geom(desc);
  if ((st = check_qtensor(dyq, mx::role_nblocks(g, MX_ROLE_GRAD))) != MX_OK) return st;
  if ((st = check_qtensor(xq, mx::role_nblocks(g, MX_ROLE_ACT))) != MX_OK) return st;
  if (!dw) return MX_ERR_NULL;
  if (!aligned(dw, 16)) return MX_ERR_ALIGN;
  if (mx::wgrad_workspace_bytes(g) > MX_NOALLOC_SCRATCH_BYTES) return MX_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MX_ERR_LAUNCH;
  return launched(mx::launch_conv_wgrad(g, dyq, xq, dw, ws, stream));
}

const char* mx_status_str(mx_status s) {
  switch (s) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "null pointer argument";
    case MX_ERR_SHAPE: return "invalid shape (dimensions, stride, padding, or C_in/C_out/N not multiples of 8)";
    case MX_ERR_FORMAT: return "unknown element format, or a format this call does not take";
    case MX_ERR_BLOCK: return "block size must be 8 or 32 (and 8 for the producer-fused amax)";
    case MX_ERR_ALIGN: return "misaligned pointer";
    case MX_ERR_WORKSPACE: return "workspace missing or smaller than mx_wgrad_workspace_bytes()";
    case MX_ERR_ROLE: return "unknown tensor role";
    case MX_ERR_LAUNCH: return "HIP launch failure";
    case MX_ERR_ROUND: return "unknown rounding mode";
  }
  return "unknown status";
}

}  // extern "C"
