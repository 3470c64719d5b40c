/*
 * mxconv.h -- C ABI of the MicroQonv microscaling convolution hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "MicroQonv: Reshaping Convolution Tensors for
 * Efficient Microscaling in Training and Inference" (Facq, Ben Ali, Sentieys;
 * arXiv 2609.28358).  Each convolution tensor is quantized exactly once, in
 * square 8x8 blocks, into a channel-batch-first layout, and the same quantized
 * tensors feed the three training GEMMs through an implicit im2col that never
 * reaches device memory (§IV-A, §IV-B).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument except the descriptor and mx_qtensor structs
 *   themselves (which live in host memory) is a DEVICE pointer.  The caller
 *   allocates and owns all buffers; the library allocates nothing and may be
 *   called from several host threads.  Its only global state is the
 *   static workspace of mx_conv_wgrad_noalloc (see there).
 * - fp32 tensors and code buffers must be 16-byte aligned; scale buffers,
 *   tensor_scale and amax 4-byte aligned.  Sources and destinations must not
 *   overlap.
 * - Arguments are validated synchronously on the host before anything is
 *   enqueued; a negative mx_status is returned and nothing runs.  On MX_OK the
 *   work has been enqueued on `stream` (asynchronous; 0 = null stream).
 *   MX_ERR_LAUNCH reports a HIP launch error.
 * - Layouts (N, the batch, is always the fastest index):
 *     activation X, its gradient dX ........ fp32 [H][W][C_in][N]
 *     output Y, output gradient dY ......... fp32 [Ho][Wo][C_out][N]
 *     weight W (FP32 master copy), dW ...... fp32 OIHW [C_out][C_in][K_h][K_w]
 *   with Ho = (H + 2 pad_h - K_h) / stride_h + 1 (likewise Wo).  The
 *   convolution is a cross-correlation with zero padding.
 * - Quantized tensors (mx_qtensor) are stored block by block:
 *     ACT    blocks [H][W][C_in/8][N/8],    in-block order [c][n]
 *     GRAD   blocks [Ho][Wo][C_out/8][N/8], in-block order [c][n]
 *     WEIGHT blocks [K_h][K_w][C_out/8][C_in/8], in-block order [co][ci]
 *   codes: E2M1 2 per byte (element 2j in the low nibble), E2M3 and E3M2 a
 *   little-endian 6-bit stream (48 bytes per block), E4M3 1 byte each; the
 *   sign is the top bit of each code.  scales: one E4M3 byte per block, in
 *   block order; the buffer continues, from the next multiple of 16 bytes,
 *   with 2 KiB that mx_quantize_cbf uses as scratch for its amax reduction
 *   (mx_scale_bytes() counts both; the GEMMs may read the scales as aligned
 *   4-byte words, which stay below that multiple of 16).  tensor_scale: one
 *   fp32.  amax: one fp32, max |x|.
 * - C_in, C_out and N must be multiples of 8 (zero-pad otherwise: padding
 *   changes neither the amax nor any result) and block must be 8.  N may be 0.
 * - block = 32 selects the original microscaling format instead (§II-D: a
 *   power-of-two E8M0 scale per block and no tensor scale; §IV-B: MicroQonv
 *   holds for any block scale), on 32x32 square blocks in the same order
 *   (ACT blocks [H][W][C_in/32][N/32], and so on), E2M1 elements throughout.
 *   C_in, C_out and N must then be multiples of 32.  A block's codes are 32
 *   rows of 16 bytes (element 2j of a row in the low nibble of byte j);
 *   scales hold one E8M0 byte per block (code e + 127 for 2^e, 0xFF NaN) and
 *   no quantizer scratch; tensor_scale is written as 1 and amax is not
 *   written.  The GEMMs run on the scaled FP4 MFMA.
 */
#ifndef MXCONV_H
#define MXCONV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = -1,      /* a required pointer is NULL */
  MX_ERR_SHAPE = -2,     /* bad dimension, stride, padding, or not a multiple of 8 */
  MX_ERR_FORMAT = -3,    /* unknown element format, or one this call does not take */
  MX_ERR_BLOCK = -4,     /* block size other than 8 or 32 (or 32 where a call takes 8 only) */
  MX_ERR_ALIGN = -5,     /* misaligned pointer */
  MX_ERR_WORKSPACE = -6, /* workspace missing or too small */
  MX_ERR_ROLE = -7,      /* unknown tensor role */
  MX_ERR_LAUNCH = -8,    /* HIP reported a launch error */
  MX_ERR_ROUND = -9      /* unknown rounding mode */
} mx_status;

/* Element formats; the block scale is always E4M3 and the tensor scale fp32
 * (the NVFP4-style two-level scaling of §II-D / §III-A, with FP6 and FP8
 * element variants of §IV-D, §IV-E and §VI-B).  MX_E3M2 is the FP6 with the
 * wider range (max 28, subnormal step 1/16): MicroQonv+ (§IV-D, Table VI)
 * keeps activations in it while weights and gradients stay E2M1 (see
 * mx_conv_desc.act_fmt).
 * MX_UE2M1 is the compact storage format of post-ReLU activations (§VI-A: the
 * sign bit removed, 3 bits per element + 8/64 for the block scale = 3.125;
 * §VII stores the latent-replay buffer so): quantized exactly like E2M1 with
 * the sign dropped (a negative element keeps its magnitude), packed as a
 * little-endian 3-bit stream, 24 bytes per block.  It is an activation
 * format only: mx_quantize_cbf and mx_dequantize take it for MX_ROLE_ACT,
 * and return MX_ERR_FORMAT for the other roles when it is elem_fmt; every
 * GEMM call that would read it returns MX_ERR_FORMAT. */
typedef enum { MX_E2M1 = 1, MX_E2M3 = 2, MX_E4M3 = 3, MX_UE2M1 = 4, MX_E3M2 = 5 } mx_elem_fmt;

/* Which tensor of the layer a quantization applies to (§IV-B: activations
 * blocked over (C_in, N), weights over (C_out, C_in), output gradients over
 * (C_out, N)). */
typedef enum { MX_ROLE_ACT = 0, MX_ROLE_WEIGHT = 1, MX_ROLE_GRAD = 2 } mx_role;

/* Element rounding (§III-A: nearest for activations and weights, stochastic
 * for gradients). */
typedef enum { MX_RNE = 0, MX_SR = 1 } mx_round;

/* One convolution layer (the problem statement of §II-A). */
typedef struct {
  int32_t n, c_in, c_out, h, w, k_h, k_w, stride_h, stride_w, pad_h, pad_w;
  int32_t elem_fmt; /* mx_elem_fmt of weights and output gradients */
  int32_t block;    /* 8 (8x8 blocks, E4M3 scale, fp32 tensor scale, §IV-B) or 32 (E8M0, see above) */
  int32_t act_fmt;  /* mx_elem_fmt of the activation X; 0 = elem_fmt */
} mx_conv_desc;
/* Format pairs the GEMMs take: elem_fmt == act_fmt (any format but
 * MX_UE2M1), or elem_fmt MX_E2M1 with act_fmt MX_E2M3 or MX_E3M2 (FP4
 * weights and gradients with FP6 activations, MicroQonv+).  mx_conv_dgrad
 * reads no activation and needs only elem_fmt to be a GEMM format; the other
 * GEMM calls, mx_wgrad_workspace_bytes and mx_fwd_amax_bytes check the pair
 * (MX_ERR_FORMAT, or 0 bytes). */

/* A quantized tensor: device pointers owned by the caller. */
typedef struct {
  void* codes;         /* packed element codes, mx_code_bytes() bytes */
  uint8_t* scales;     /* E4M3 block scales + amax scratch, mx_scale_bytes() bytes */
  float* tensor_scale; /* one fp32: T */
  float* amax;         /* one fp32: max |x| of the source */
} mx_qtensor;

/* Bytes of the codes / scales buffers of the tensor of `role`, in that
 * role's format (act_fmt for MX_ROLE_ACT) (0 on an invalid descriptor or
 * role).  The scales buffer holds ceil-to-16 of the
 * block count bytes of scales plus 2048 bytes of quantizer scratch (0 bytes
 * in all for an empty tensor). */
size_t mx_code_bytes(const mx_conv_desc* desc, mx_role role);
size_t mx_scale_bytes(const mx_conv_desc* desc, mx_role role);

/* Bytes of device workspace mx_conv_wgrad needs for this layer (0 on an
 * invalid descriptor). */
size_t mx_wgrad_workspace_bytes(const mx_conv_desc* desc);

/* Quantize one fp32 tensor into 8x8 microscaling blocks (§III-A, §IV-B).
 *   T     = amax / (448 * max_elem)
 *   B     = E4M3_RNE_sat(blockamax / (max_elem * T))      one per 8x8 block
 *   code  = Round(|x| / (B * T)) on the element grid, sign = sign of x
 * Round is nearest-even (MX_RNE) or stochastic (MX_SR): round up iff
 * u * (hi - lo) < v - lo, where u takes 24 bits of
 * h = SplitMix64(seed ^ 0x9E3779B97F4A7C15 * (i/2 + 1)): bits 40..63 of h for
 * an even i, bits 16..39 for an odd i, with i the element's linear index in
 * `src`.  Every fp32 step is one correctly rounded IEEE operation.
 *   src        fp32 tensor of `role` in the layout above
 *   dst        quantized tensor: codes, scales, tensor_scale and amax written;
 *              codes and scales 16-byte aligned.  The amax pass keeps one
 *              partial maximum per workgroup in the scratch tail of the
 *              scales buffer, so no atomics and no zero-fill are needed
 *   amax_given 0: *dst->amax is computed here (max |x|, two passes over src);
 *              1: *dst->amax already holds the amax to use (e.g. a
 *              statistic carried over from a previous step); not written
 * Non-finite input (Inf/NaN, or a non-finite given amax) is reported in-band:
 * *tensor_scale = NaN, every scale byte 0x7F (E4M3 NaN), all codes 0.
 * With block = 32 (E8M0 scales, one pass over src, amax_given ignored):
 *   e     = floor(log2 blockamax) - 2, clamped to [-127, 127]  (OCP MX rule)
 *   code  = Round(|x| / 2^e) on the E2M1 grid, saturating, sign of x
 *   scale byte e + 127; 0 for an all-zero block; a block holding Inf or NaN
 *   gets scale 0xFF and codes 0 (other blocks are unaffected). */
mx_status mx_quantize_cbf(const mx_conv_desc* desc, mx_role role, const float* src,
                          const mx_qtensor* dst, mx_round rounding, uint64_t seed,
                          int amax_given, hipStream_t stream);

/* Forward convolution Y = W_f . X' (§II-C, §IV-B) with X' the channel-batch-
 * first im2col of the quantized activation, formed on chip only.
 *   wq  quantized weight (role WEIGHT), xq quantized activation (role ACT)
 *   y   fp32 [Ho][Wo][C_out][N], overwritten
 * Products of dequantized elements are exact; sums are fp32. */
mx_status mx_conv_fwd(const mx_conv_desc* desc, const mx_qtensor* wq, const mx_qtensor* xq,
                      float* y, hipStream_t stream);

/* mx_conv_fwd that also produces max |y| over every output element (§VII
 * loads each tensor once with its statistic estimated ahead of time; here
 * the producer supplies the exact statistic instead).  Passing y_amax as the
 * amax of the next quantization of y (amax_given = 1) then skips that
 * call's amax pass: one read of y instead of two, with the same codes.
 *   y_amax device buffer of mx_fwd_amax_bytes(desc) bytes, 4-byte aligned;
 *          y_amax[0] is overwritten with max |y| (the comparison is the
 *          unsigned order of the sign-cleared bits, so a NaN in y gives a
 *          NaN amax, which quantizes as non-finite input); the rest of the
 *          buffer receives one partial maximum per wave of the GEMM (no
 *          atomics), so its contents are unspecified
 * Errors as mx_conv_fwd, plus MX_ERR_NULL / MX_ERR_ALIGN for y_amax, and
 * MX_ERR_BLOCK for block = 32 (no tensor amax there; mx_fwd_amax_bytes
 * returns 0). */
size_t mx_fwd_amax_bytes(const mx_conv_desc* desc);
mx_status mx_conv_fwd_amax(const mx_conv_desc* desc, const mx_qtensor* wq, const mx_qtensor* xq,
                           float* y, float* y_amax, hipStream_t stream);

/* Data gradient dX = col2im(W_f^T . dY) (§II-A "transposed kernels",
 * §IV-B), evaluated in gather form: each dX element sums exactly the
 * products col2im would add into it.
 *   wq quantized weight, dyq quantized output gradient (role GRAD)
 *   dx fp32 [H][W][C_in][N], overwritten */
mx_status mx_conv_dgrad(const mx_conv_desc* desc, const mx_qtensor* wq, const mx_qtensor* dyq,
                        float* dx, hipStream_t stream);

/* Weight gradient dW = dY . X'^T accumulated over the batch (§II-A, §IV-B).
 *   dyq quantized output gradient, xq quantized activation
 *   dw        fp32 OIHW, overwritten
 *   workspace device buffer of at least mx_wgrad_workspace_bytes(desc) bytes
 *             (partial sums of the split reduction; contents on return are
 *             unspecified).  The reduction order is fixed: results are
 *             bit-reproducible run to run. */
mx_status mx_conv_wgrad(const mx_conv_desc* desc, const mx_qtensor* dyq, const mx_qtensor* xq,
                        float* dw, void* workspace, size_t ws_bytes, hipStream_t stream);

/* mx_conv_wgrad for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The split partials go to a static array in device memory that the library
 * holds on each GPU it runs on, MX_NOALLOC_SCRATCH_BYTES bytes (64 MiB,
 * enough for every layer of the five workloads this library is measured
 * on: 63 MiB at most), until the process ends; the call allocates nothing
 * and calls no allocating routine.  The first call on a device looks up
 * that device's copy (once; cached).
 *   dyq, xq, dw as for mx_conv_wgrad; the result is bit-identical to it
 *   (same kernels, same split plan, same reduction order)
 * Errors as mx_conv_wgrad, except that there is no workspace argument:
 * MX_ERR_WORKSPACE when the layer needs more than MX_NOALLOC_SCRATCH_BYTES
 * (mx_wgrad_workspace_bytes(desc) tells); MX_ERR_LAUNCH also when the
 * array's address cannot be obtained.  Every call on one GPU shares that
 * GPU's array and the partials are written before they are read, so nothing
 * needs clearing between calls, but calls that overlap in time on one GPU
 * (concurrent streams, or host threads) race on it: serialize them. */
#define MX_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mx_status mx_conv_wgrad_noalloc(const mx_conv_desc* desc, const mx_qtensor* dyq, const mx_qtensor* xq,
                                float* dw, hipStream_t stream);

/* Explicit channel-batch-first im2col: the expanded activation X' that the
 * quantize-after-im2col flow (§III-C, the extrapolation of Cuyckens et al.
 * to convolutions; Table I) writes to memory and MicroQonv never forms.
 *   x     fp32 [H][W][C_in][N]
 *   xcol  fp32 [Ho][Wo][Kh][Kw][C_in][N], overwritten; zero where a tap falls
 *         in the padding.  As an activation it is a 1x1 convolution input
 *         with C_in' = Kh*Kw*C_in channels on an Ho x Wo image, so the
 *         baseline flow is mx_im2col_cbf + mx_quantize_cbf + the GEMM calls
 *         on that 1x1 descriptor.
 * Pointers 16-byte aligned; errors as the other calls. */
mx_status mx_im2col_cbf(const mx_conv_desc* desc, const float* x, float* xcol, hipStream_t stream);

/* Fake-quantized fp32 values (-1)^s * fl32(fl32(g * B) * T) (§III-A), written
 * in the fp32 layout of `role`. */
mx_status mx_dequantize(const mx_conv_desc* desc, mx_role role, const mx_qtensor* q, float* dst,
                        hipStream_t stream);

/* Static description of a status code. */
const char* mx_status_str(mx_status status);

#ifdef __cplusplus
}
#endif

#endif /* MXCONV_H */
