/*
 * mxconv_oracle.c -- plain, slow CPU oracle for the MicroQonv hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP implementation: every format grid, rounding rule and index mapping
 * below is written out again from the paper's description.
 *
 * Source: "MicroQonv: Reshaping Convolution Tensors for Efficient Microscaling
 * in Training and Inference" (Facq, Ben Ali, Sentieys; arXiv 2609.28358).
 *
 *   - two-level NVFP4-style scaling (per-tensor FP32 scale T, per-block E4M3
 *     scale B, element Round(.)), round-to-nearest for activations/weights and
 *     stochastic rounding for gradients ............ §II-D and §III-A
 *   - square 8x8 (B = 64) blocks; activations blocked over (C_in, N), weights
 *     over (C_out, C_in), output gradients over (C_out, N) ..... §IV-B
 *   - channel-batch-first activation layout X_{Cin,N}: each spatial position
 *     holds one contiguous (C, N) plane ............ §IV-A, Fig. 3
 *   - im2col matrix X' (rows = kernel position x channel, columns = output
 *     window x batch) and the three GEMMs Y = W X', G_W = G_Y X'^T,
 *     G_X' = W^T G_Y followed by col2im ............ §II-C, §IV-B
 *   - per-element quantization counts of Table I (MicroQonv x1, quantize-
 *     after-im2col x9, DaCapo x18) ................. §IV-C, Table I
 *
 * Readings where the pages are silent or garbled (their display equations
 * were lost in extraction; only the "where" clauses survive):
 *   T     = fl32(amax / (maxBsf * maxBef))              (0 if amax == 0)
 *   B_raw = fl32(a_i / fl32(maxBef * T))                (0 if T == 0)
 *   B     = E4M3 round-to-nearest-even, saturating at 448
 *   v     = fl32(|x| / fl32(B * T))                     (0 if B*T == 0)
 *   code  = element grid round-to-nearest-even (ties to the even code),
 *           saturating; sign bit = signbit(x)
 *   stochastic rounding: lo <= v < hi adjacent grid points, round up iff
 *           u * (hi - lo) < v - lo, u = 24 bits of h = SplitMix64 (Steele,
 *           Lea & Flood, OOPSLA 2014) of seed ^ (0x9E3779B97F4A7C15*(idx/2+1))
 *           (bits 40..63 of h for even idx, bits 16..39 for odd idx), idx the
 *           element's linear index in the fp32 source
 *   non-finite input: T = NaN, every block scale 0x7F (E4M3 NaN), codes 0
 *
 * All fp32 steps are single IEEE operations (build with -ffp-contract=off, no
 * fast-math).  The GEMMs run in fp64 on the exact dequantized values
 * (q * B * T is exact in fp64: at most 8 + 24 significant bits).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E2M1 1
#define ORC_E2M3 2
#define ORC_E4M3 3
#define ORC_E3M2 4
/* E2M1 magnitude without the sign bit: the 3-bit activation codes of a
 * post-ReLU tensor (§VI-A: after a ReLU the sign bit carries nothing and is
 * dropped, 3 + 8/64 = 3.125 bits per element with the block scale), used by
 * the compact latent-replay
 * buffer (§VII).  Quantized like E2M1; a negative element keeps only its
 * magnitude. */
#define ORC_UE2M1 5

#define ORC_ACT 0
#define ORC_WEIGHT 1
#define ORC_GRAD 2

#define ORC_RNE 0
#define ORC_SR 1

/* ------------------------------------------------------------------------ */
/* Element and scale formats (OCP microscaling conventions: sign | exponent |  */
/* mantissa, subnormals when the exponent field is 0; E4M3 "fn" has no         */
/* infinity and uses S.1111.111 for NaN, so its largest finite value is 448;   */
/* E2M1's largest value is 6 -- the two maxima the paper's §III-A names).      */
/* ------------------------------------------------------------------------ */

typedef struct {
  int ebits, mbits, bias;
  int nmag;   /* number of finite magnitude codes */
  int signed_; /* 1: a sign bit above the magnitude; 0: magnitude only */
} orc_fmt_t;

static int fmt_desc(int fmt, orc_fmt_t* f) {
  switch (fmt) {
    case ORC_E2M1: f->ebits = 2; f->mbits = 1; f->bias = 1; f->nmag = 8; f->signed_ = 1; return 0;
    case ORC_E2M3: f->ebits = 2; f->mbits = 3; f->bias = 1; f->nmag = 32; f->signed_ = 1; return 0;
    case ORC_E3M2: f->ebits = 3; f->mbits = 2; f->bias = 3; f->nmag = 32; f->signed_ = 1; return 0;
    case ORC_E4M3: f->ebits = 4; f->mbits = 3; f->bias = 7; f->nmag = 127; f->signed_ = 1; return 0;
    case ORC_UE2M1: f->ebits = 2; f->mbits = 1; f->bias = 1; f->nmag = 8; f->signed_ = 0; return 0;
    default: return -1;
  }
}

/* Real value of a magnitude code (exact in double). */
double orc_fmt_value(int fmt, int mag) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f) || mag < 0 || mag >= f.nmag) return NAN;
  int e = mag >> f.mbits;
  int m = mag & ((1 << f.mbits) - 1);
  double frac = (double)m / (double)(1 << f.mbits);
  if (e == 0) return ldexp(frac, 1 - f.bias);
  return ldexp(1.0 + frac, e - f.bias);
}

int orc_fmt_nmag(int fmt) {
  orc_fmt_t f;
  return fmt_desc(fmt, &f) ? -1 : f.nmag;
}

int orc_fmt_sign_shift(int fmt) {
  orc_fmt_t f;
  return fmt_desc(fmt, &f) ? -1 : f.ebits + f.mbits;
}

int orc_fmt_bits(int fmt) {
  orc_fmt_t f;
  return fmt_desc(fmt, &f) ? -1 : f.signed_ + f.ebits + f.mbits;
}

double orc_fmt_max(int fmt) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f)) return NAN;
  return orc_fmt_value(fmt, f.nmag - 1);
}

/* Largest magnitude code whose value is <= v (v >= 0, finite). Binary search
 * over the ascending grid. */
static int grid_floor(int fmt, int nmag, double v) {
  int lo = 0, hi = nmag - 1; /* invariant: value(lo) <= v */
  if (orc_fmt_value(fmt, hi) <= v) return hi;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_fmt_value(fmt, mid) <= v) lo = mid; else hi = mid;
  }
  return lo;
}

/* Round-to-nearest, ties to the even code, saturating at the format maximum.
 * v must be >= 0 (magnitude).  NaN is not accepted (returns -1). */
int orc_round_rne(int fmt, float v) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f) || !(v >= 0.0f)) return -1;
  double dv = (double)v;
  int lo = grid_floor(fmt, f.nmag, dv);
  if (lo == f.nmag - 1) return lo; /* at or above the maximum: saturate */
  double a = orc_fmt_value(fmt, lo), b = orc_fmt_value(fmt, lo + 1);
  double dlo = dv - a, dhi = b - dv; /* exact: all operands have <= 24 bits */
  if (dlo < dhi) return lo;
  if (dhi < dlo) return lo + 1;
  return (lo % 2 == 0) ? lo : lo + 1;
}

/* Stochastic rounding: round up iff u*(hi-lo) < v-lo, evaluated in fp32.
 * Both fp32 operations are exact (Sterbenz for the difference, power-of-two
 * spacing for the product), so the decision is reproducible. */
int orc_round_sr(int fmt, float v, float u) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f) || !(v >= 0.0f)) return -1;
  int lo = grid_floor(fmt, f.nmag, (double)v);
  if (lo == f.nmag - 1) return lo;
  float a = (float)orc_fmt_value(fmt, lo);
  float b = (float)orc_fmt_value(fmt, lo + 1);
  float delta = b - a;
  float diff = v - a;
  float thr = u * delta;
  return (thr < diff) ? lo + 1 : lo;
}

/* SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). */
uint64_t orc_splitmix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Uniform in [0,1) with 24 random bits, for element index idx: elements
 * 2k and 2k+1 share the SplitMix64 output of counter k, the even one taking
 * its bits 40..63, the odd one its bits 16..39. */
float orc_sr_uniform(uint64_t seed, uint64_t idx) {
  uint64_t h = orc_splitmix64(seed ^ (0x9E3779B97F4A7C15ULL * ((idx >> 1) + 1ULL)));
  uint64_t bits = (idx & 1ULL) ? ((h >> 16) & 0xFFFFFFULL) : (h >> 40);
  return (float)bits * (1.0f / 16777216.0f);
}

/* ------------------------------------------------------------------------ */
/* Tensor roles and block geometry (§IV-A, §IV-B).                             */
/*   ACT  : fp32 source [H][W][C][N]   blocks (h, w, C/8, N/8), block [c][n]   */
/*   GRAD : fp32 source [Ho][Wo][C][N] same geometry with C = C_out           */
/*   WEIGHT: fp32 source OIHW [Co][Ci][Kh][Kw]                                 */
/*          blocks (kh, kw, Co/8, Ci/8), block [co][ci]                        */
/* Dimensions are passed as (d0, d1, d2, d3) = (H, W, C, N) or (Co, Ci, Kh, Kw)*/
/* ------------------------------------------------------------------------ */

static int64_t role_nblocks(int role, const int64_t d[4]) {
  if (role == ORC_WEIGHT) return d[2] * d[3] * (d[0] / 8) * (d[1] / 8);
  return d[0] * d[1] * (d[2] / 8) * (d[3] / 8);
}

/* Linear index in the fp32 source of element (r, c) of block b. */
static int64_t role_src_index(int role, const int64_t d[4], int64_t b, int r, int c) {
  if (role == ORC_WEIGHT) {
    int64_t Co = d[0], Ci = d[1], Kh = d[2], Kw = d[3];
    int64_t cib = b % (Ci / 8);
    int64_t t = b / (Ci / 8);
    int64_t cob = t % (Co / 8);
    t /= (Co / 8);
    int64_t kw = t % Kw, kh = t / Kw;
    int64_t co = cob * 8 + r, ci = cib * 8 + c;
    return ((co * Ci + ci) * Kh + kh) * Kw + kw;
  } else {
    int64_t W = d[1], C = d[2], N = d[3];
    int64_t nb = b % (N / 8);
    int64_t t = b / (N / 8);
    int64_t cb = t % (C / 8);
    int64_t p = t / (C / 8); /* spatial position h*W + w */
    (void)W;
    return (p * C + cb * 8 + r) * N + nb * 8 + c;
  }
}

int64_t orc_role_nblocks(int role, int64_t d0, int64_t d1, int64_t d2, int64_t d3) {
  int64_t d[4] = {d0, d1, d2, d3};
  return role_nblocks(role, d);
}

int64_t orc_role_src_index(int role, int64_t d0, int64_t d1, int64_t d2, int64_t d3,
                           int64_t b, int r, int c) {
  int64_t d[4] = {d0, d1, d2, d3};
  return role_src_index(role, d, b, r, c);
}

static float fmt_max_f(int fmt) { return (float)orc_fmt_max(fmt); }

/* E4M3 cast of a non-negative block scale: nearest-even, saturating. */
int orc_e4m3_code(float v) { return orc_round_rne(ORC_E4M3, v); }

/* The per-tensor amax: max |x|; *nonfinite set if any element is Inf/NaN
 * (then amax is NaN when a NaN is present, +Inf otherwise). */
float orc_amax(const float* src, int64_t n, int* nonfinite) {
  float m = 0.0f;
  int has_nan = 0, has_inf = 0;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(src[i]);
    if (isnan(a)) has_nan = 1;
    else if (isinf(a)) has_inf = 1;
    else if (a > m) m = a;
  }
  *nonfinite = has_nan || has_inf;
  if (has_nan) return NAN;
  if (has_inf) return INFINITY;
  return m;
}

/* Quantize one tensor (O2-O5).
 *   codes : one byte per element, in block order (block b, then row, col);
 *           magnitude code in the low bits, sign at bit (ebits+mbits)
 *   scales: one E4M3 byte per block
 * If amax_in is non-NULL its value is used as the tensor amax instead of
 * scanning src (the caller-supplied statistic).  Returns 0 or -1. */
int orc_quantize(int role, int fmt, int rounding, uint64_t seed, const float* src,
                 int64_t d0, int64_t d1, int64_t d2, int64_t d3, const float* amax_in,
                 uint8_t* codes, uint8_t* scales, float* t_out, float* amax_out) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f)) return -1;
  int64_t d[4] = {d0, d1, d2, d3};
  if (role == ORC_WEIGHT) {
    if (d0 % 8 || d1 % 8) return -1;
  } else if (role == ORC_ACT || role == ORC_GRAD) {
    if (d2 % 8 || d3 % 8) return -1;
  } else {
    return -1;
  }
  int64_t nel = d0 * d1 * d2 * d3;
  int64_t nb = role_nblocks(role, d);
  int sign_shift = f.ebits + f.mbits;

  int nonfinite = 0;
  float amax;
  if (amax_in) {
    /* a caller-supplied statistic is used by magnitude and reported as given */
    *amax_out = *amax_in;
    amax = fabsf(*amax_in);
    nonfinite = !isfinite(amax);
  } else {
    amax = orc_amax(src, nel, &nonfinite);
    *amax_out = amax;
  }
  if (nonfinite) {
    *t_out = NAN;
    memset(scales, 0x7F, (size_t)nb);
    memset(codes, 0, (size_t)nel);
    return 0;
  }
  const float maxBsf = 448.0f;           /* E4M3 */
  const float maxBef = fmt_max_f(fmt);   /* 6, 7.5, 448 (28 for E3M2) */
  const float K = maxBsf * maxBef;       /* exact */
  float T = amax / K;
  if (amax == 0.0f) T = 0.0f;
  *t_out = T;
  float den = maxBef * T;

#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    float ai = 0.0f;
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) {
        float a = fabsf(src[role_src_index(role, d, b, r, c)]);
        if (a > ai) ai = a;
      }
    float braw = (T == 0.0f) ? 0.0f : ai / den;
    int bcode = orc_e4m3_code(braw);
    float B = (float)orc_fmt_value(ORC_E4M3, bcode);
    scales[b] = (uint8_t)bcode;
    float dd = B * T;
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) {
        int64_t si = role_src_index(role, d, b, r, c);
        float x = src[si];
        float v = (dd == 0.0f) ? 0.0f : fabsf(x) / dd;
        int mag;
        if (rounding == ORC_SR) mag = orc_round_sr(fmt, v, orc_sr_uniform(seed, (uint64_t)si));
        else mag = orc_round_rne(fmt, v);
        int s = (f.signed_ && signbit(x)) ? 1 : 0; /* an unsigned format drops the sign */
        codes[b * 64 + r * 8 + c] = (uint8_t)(mag | (s << sign_shift));
      }
  }
  return 0;
}

/* Quantize only the listed blocks, given the tensor amax (for sampled checks
 * of very large tensors).  codes: 64 bytes per listed block. */
int orc_quantize_blocks(int role, int fmt, int rounding, uint64_t seed, const float* src,
                        int64_t d0, int64_t d1, int64_t d2, int64_t d3, float amax,
                        const int64_t* blocks, int64_t nsel, uint8_t* codes, uint8_t* scales,
                        float* t_out) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f)) return -1;
  int64_t d[4] = {d0, d1, d2, d3};
  int sign_shift = f.ebits + f.mbits;
  if (!isfinite(amax)) {
    *t_out = NAN;
    memset(scales, 0x7F, (size_t)nsel);
    memset(codes, 0, (size_t)nsel * 64);
    return 0;
  }
  const float maxBef = fmt_max_f(fmt);
  const float K = 448.0f * maxBef;
  float T = amax / K;
  if (amax == 0.0f) T = 0.0f;
  *t_out = T;
  float den = maxBef * T;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nsel; ++i) {
    int64_t b = blocks[i];
    float ai = 0.0f;
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) {
        float a = fabsf(src[role_src_index(role, d, b, r, c)]);
        if (a > ai) ai = a;
      }
    float braw = (T == 0.0f) ? 0.0f : ai / den;
    int bcode = orc_e4m3_code(braw);
    float B = (float)orc_fmt_value(ORC_E4M3, bcode);
    scales[i] = (uint8_t)bcode;
    float dd = B * T;
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) {
        int64_t si = role_src_index(role, d, b, r, c);
        float x = src[si];
        float v = (dd == 0.0f) ? 0.0f : fabsf(x) / dd;
        int mag = (rounding == ORC_SR) ? orc_round_sr(fmt, v, orc_sr_uniform(seed, (uint64_t)si))
                                       : orc_round_rne(fmt, v);
        codes[i * 64 + r * 8 + c] = (uint8_t)(mag | (((f.signed_ && signbit(x)) ? 1 : 0) << sign_shift));
      }
  }
  return 0;
}

/* Magnitude value, sign and block scale of one code -> signed real value of
 * code * B (exact in double). */
static double code_times_scale(int fmt, int sign_shift, uint8_t code, uint8_t scale) {
  if (scale == 0x7F) return NAN;
  int mag = code & ((1 << sign_shift) - 1);
  double v = orc_fmt_value(fmt, mag) * orc_fmt_value(ORC_E4M3, scale);
  return (code >> sign_shift) & 1 ? -v : v;
}

/* Fake-quantized fp32 value (O7): (-1)^s * fl32(fl32(g*B) * T), written into
 * the role's fp32 layout. */
int orc_dequantize(int role, int fmt, int64_t d0, int64_t d1, int64_t d2, int64_t d3,
                   const uint8_t* codes, const uint8_t* scales, float T, float* dst) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f)) return -1;
  int64_t d[4] = {d0, d1, d2, d3};
  int64_t nb = role_nblocks(role, d);
  int sign_shift = f.ebits + f.mbits;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    uint8_t s = scales[b];
    float B = (s == 0x7F) ? NAN : (float)orc_fmt_value(ORC_E4M3, s);
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c) {
        uint8_t code = codes[b * 64 + r * 8 + c];
        float g = (float)orc_fmt_value(fmt, code & ((1 << sign_shift) - 1));
        float gb = g * B;
        float v = gb * T;
        if ((code >> sign_shift) & 1) v = -v;
        dst[role_src_index(role, d, b, r, c)] = v;
      }
  }
  return 0;
}

/* Exact dequantized values q*B*T in fp64, in the role's fp32 layout. */
int orc_dequantize64(int role, int fmt, int64_t d0, int64_t d1, int64_t d2, int64_t d3,
                     const uint8_t* codes, const uint8_t* scales, float T, double* dst) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f)) return -1;
  int64_t d[4] = {d0, d1, d2, d3};
  int64_t nb = role_nblocks(role, d);
  int sign_shift = f.ebits + f.mbits;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b)
    for (int r = 0; r < 8; ++r)
      for (int c = 0; c < 8; ++c)
        dst[role_src_index(role, d, b, r, c)] =
            code_times_scale(fmt, sign_shift, codes[b * 64 + r * 8 + c], scales[b]) * (double)T;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The original microscaling format (§II-D: a power-of-two block scale in   */
/* E8M0, no tensor scale) on square S x S blocks in the same channel-batch- */
/* first block order (§IV-A, §IV-B: MicroQonv holds for any block scale).   */
/* The shared scale of a block is 2^e with e = floor(log2 amax_block) minus  */
/* the exponent of the element format's largest value (the OCP MX rule),    */
/* clamped to the E8M0 range [-127, 127]; each element is |x| / 2^e rounded  */
/* onto the element grid (saturating), sign kept.                           */
/* ------------------------------------------------------------------------ */

static int64_t mx_nblocks(int role, const int64_t d[4], int S) {
  if (role == ORC_WEIGHT) return d[2] * d[3] * (d[0] / S) * (d[1] / S);
  return d[0] * d[1] * (d[2] / S) * (d[3] / S);
}

/* Source index of element (r, c) of block b: blocks [H][W][C/S][N/S] with
 * (r, c) = (channel, sample) for activations and gradients, blocks
 * [Kh][Kw][Co/S][Ci/S] with (r, c) = (co, ci) for weights. */
static int64_t mx_src_index(int role, const int64_t d[4], int S, int64_t b, int r, int c) {
  if (role == ORC_WEIGHT) {
    int64_t Co = d[0], Ci = d[1], Kh = d[2], Kw = d[3];
    int64_t cib = b % (Ci / S), t = b / (Ci / S);
    int64_t cob = t % (Co / S);
    t /= (Co / S);
    int64_t kw = t % Kw, kh = t / Kw;
    return (((cob * S + r) * Ci + cib * S + c) * Kh + kh) * Kw + kw;
  }
  int64_t C = d[2], N = d[3];
  int64_t nb = b % (N / S), t = b / (N / S);
  int64_t cb = t % (C / S), pos = t / (C / S);
  return (pos * C + cb * S + r) * N + nb * S + c;
}

int64_t orc_mx_nblocks(int role, int S, int64_t d0, int64_t d1, int64_t d2, int64_t d3) {
  int64_t d[4] = {d0, d1, d2, d3};
  return mx_nblocks(role, d, S);
}
int64_t orc_mx_src_index(int role, int S, int64_t d0, int64_t d1, int64_t d2, int64_t d3, int64_t b, int r,
                         int c) {
  int64_t d[4] = {d0, d1, d2, d3};
  return mx_src_index(role, d, S, b, r, c);
}

/* floor(log2 a) for a finite a > 0, from the binary exponent (exact). */
static int floor_log2f(float a) {
  int e;
  frexpf(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  return e - 1;
}

/* E8M0 code of the shared scale of a block with maximum magnitude amax:
 * 0xFF when the block holds a non-finite value, 0 (2^-127) for an all-zero
 * block. */
int orc_e8m0_code(int fmt, float amax, int nonfinite) {
  if (nonfinite) return 0xFF;
  if (amax == 0.0f) return 0;
  int e = floor_log2f(amax) - floor_log2f(fmt_max_f(fmt));
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e + 127;
}

/* Quantize one tensor in S x S MX blocks: codes one byte per element in
 * block order (block, then row, column), scales one E8M0 byte per block.
 * Returns 0, or -1 on a bad format, role or shape. */
int orc_quantize_mx(int role, int fmt, int rounding, uint64_t seed, int S, const float* src, int64_t d0,
                    int64_t d1, int64_t d2, int64_t d3, uint8_t* codes, uint8_t* scales) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f) || !f.signed_ || S <= 0) return -1;
  int64_t d[4] = {d0, d1, d2, d3};
  if (role == ORC_WEIGHT) {
    if (d0 % S || d1 % S) return -1;
  } else if (role == ORC_ACT || role == ORC_GRAD) {
    if (d2 % S || d3 % S) return -1;
  } else {
    return -1;
  }
  int64_t nb = mx_nblocks(role, d, S);
  int sign_shift = f.ebits + f.mbits;
  int64_t bs = (int64_t)S * S;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    float amax = 0.0f;
    int nonfinite = 0;
    for (int r = 0; r < S; ++r)
      for (int c = 0; c < S; ++c) {
        float a = fabsf(src[mx_src_index(role, d, S, b, r, c)]);
        if (!isfinite(a)) nonfinite = 1;
        else if (a > amax) amax = a;
      }
    int code = orc_e8m0_code(fmt, amax, nonfinite);
    scales[b] = (uint8_t)code;
    /* 1 / 2^e, exact for e in [-127, 127] */
    float inv = ldexpf(1.0f, 127 - code);
    for (int r = 0; r < S; ++r)
      for (int c = 0; c < S; ++c) {
        int64_t si = mx_src_index(role, d, S, b, r, c);
        float x = src[si];
        int mag = 0;
        if (!nonfinite) {
          float v = fabsf(x) * inv;
          mag = (rounding == ORC_SR) ? orc_round_sr(fmt, v, orc_sr_uniform(seed, (uint64_t)si)) : orc_round_rne(fmt, v);
        }
        int sgn = (!nonfinite && signbit(x)) ? 1 : 0;
        codes[b * bs + (int64_t)r * S + c] = (uint8_t)(mag | (sgn << sign_shift));
      }
  }
  return 0;
}

/* Exact dequantized values g * 2^e (NaN for a 0xFF scale) in the role's
 * layout, as fp64 (dst64) and/or fp32 (dst32, exact as well: the products
 * lie within fp32's range down to its subnormals). */
int orc_dequantize_mx(int role, int fmt, int S, int64_t d0, int64_t d1, int64_t d2, int64_t d3,
                      const uint8_t* codes, const uint8_t* scales, double* dst64, float* dst32) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f) || S <= 0) return -1;
  int64_t d[4] = {d0, d1, d2, d3};
  int64_t nb = mx_nblocks(role, d, S);
  int sign_shift = f.ebits + f.mbits;
  int64_t bs = (int64_t)S * S;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    double scale = scales[b] == 0xFF ? NAN : ldexp(1.0, (int)scales[b] - 127);
    for (int r = 0; r < S; ++r)
      for (int c = 0; c < S; ++c) {
        uint8_t code = codes[b * bs + (int64_t)r * S + c];
        double v = orc_fmt_value(fmt, code & ((1 << sign_shift) - 1)) * scale;
        if ((code >> sign_shift) & 1) v = -v;
        int64_t si = mx_src_index(role, d, S, b, r, c);
        if (dst64) dst64[si] = v;
        if (dst32) dst32[si] = (float)v;
      }
  }
  return 0;
}

/* Pack codes (O6): E2M1 two per byte, element 2j in the low nibble; E2M3 and
 * E3M2 as a little-endian 6-bit stream (48 bytes per 64-element block), the
 * unsigned 3-bit E2M1 as a 3-bit stream (24 bytes per block); E4M3 one byte
 * each. */
int orc_pack(int fmt, const uint8_t* codes, int64_t nel, uint8_t* out) {
  int bits = orc_fmt_bits(fmt);
  if (bits == 4) {
    for (int64_t j = 0; j < nel / 2; ++j)
      out[j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
  } else if (bits == 6 || bits == 3) {
    /* little-endian bit stream per 64-element block: element e of a block at
     * bits e*bits .. e*bits + bits - 1 */
    memset(out, 0, (size_t)(nel * bits / 8));
    for (int64_t i = 0; i < nel; ++i) {
      int64_t blk = i / 64, e = i % 64;
      for (int k = 0; k < bits; ++k) {
        int64_t bit = blk * 64 * bits + e * bits + k;
        if ((codes[i] >> k) & 1) out[bit / 8] |= (uint8_t)(1u << (bit % 8));
      }
    }
  } else if (bits == 8) {
    memcpy(out, codes, (size_t)nel);
  } else {
    return -1;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Convolution geometry, explicit im2col and fp64 GEMMs (§II-C, §IV-B).        */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n, c_in, c_out, h, w, k_h, k_w, stride_h, stride_w, pad_h, pad_w;
} orc_conv;

static int64_t out_h(const orc_conv* cv) { return (cv->h + 2 * cv->pad_h - cv->k_h) / cv->stride_h + 1; }
static int64_t out_w(const orc_conv* cv) { return (cv->w + 2 * cv->pad_w - cv->k_w) / cv->stride_w + 1; }

/* im2col row k = (kh, kw, ci) (channel fastest), column j = (ho, wo, n) (batch
 * fastest).  Returns the linear index of the referenced activation in the
 * [H][W][C][N] layout, or -1 inside the zero-padding region. */
int64_t orc_im2col_src(const orc_conv* cv, int64_t k, int64_t j) {
  int64_t Ho = out_h(cv), Wo = out_w(cv);
  int64_t ci = k % cv->c_in, tap = k / cv->c_in;
  int64_t kw = tap % cv->k_w, kh = tap / cv->k_w;
  int64_t n = j % cv->n, pos = j / cv->n;
  int64_t wo = pos % Wo, ho = pos / Wo;
  (void)Ho;
  int64_t hh = ho * cv->stride_h + kh - cv->pad_h;
  int64_t ww = wo * cv->stride_w + kw - cv->pad_w;
  if (hh < 0 || hh >= cv->h || ww < 0 || ww >= cv->w) return -1;
  return ((hh * cv->w + ww) * cv->c_in + ci) * cv->n + n;
}

/* Explicit patch matrix, stored column by column: xt[j*K + k] = X'[k][j]. */
static double* build_im2col_cols(const orc_conv* cv, const double* x) {
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = out_h(cv) * out_w(cv) * cv->n;
  double* xt = (double*)malloc(sizeof(double) * (size_t)(K * J));
  if (!xt) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < J; ++j)
    for (int64_t k = 0; k < K; ++k) {
      int64_t s = orc_im2col_src(cv, k, j);
      xt[j * K + k] = s < 0 ? 0.0 : x[s];
    }
  return xt;
}

/* Flattened weights W_f[co][k], k = (kh, kw, ci), from OIHW. */
static double* build_wf(const orc_conv* cv, const double* w) {
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  double* wf = (double*)malloc(sizeof(double) * (size_t)(cv->c_out * K));
  if (!wf) return NULL;
  for (int64_t co = 0; co < cv->c_out; ++co)
    for (int64_t kh = 0; kh < cv->k_h; ++kh)
      for (int64_t kw = 0; kw < cv->k_w; ++kw)
        for (int64_t ci = 0; ci < cv->c_in; ++ci)
          wf[co * K + (kh * cv->k_w + kw) * cv->c_in + ci] =
              w[((co * cv->c_in + ci) * cv->k_h + kh) * cv->k_w + kw];
  return wf;
}

/* Y[co][j] = sum_k W_f[co][k] X'[k][j]; written to [Ho][Wo][Co][N].
 * sabs receives sum_k |W_f X'| for the tolerance. */
int orc_conv_fwd(const orc_conv* cv, const double* w, const double* x, double* y, double* sabs) {
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = out_h(cv) * out_w(cv) * cv->n;
  double* xt = build_im2col_cols(cv, x);
  double* wf = build_wf(cv, w);
  if (!xt || !wf) { free(xt); free(wf); return -1; }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < J; ++j) {
    int64_t n = j % cv->n, pos = j / cv->n;
    for (int64_t co = 0; co < cv->c_out; ++co) {
      double acc = 0.0, sa = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = wf[co * K + k] * xt[j * K + k];
        acc += p;
        sa += fabs(p);
      }
      int64_t o = (pos * cv->c_out + co) * cv->n + n;
      y[o] = acc;
      sabs[o] = sa;
    }
  }
  free(xt);
  free(wf);
  return 0;
}

/* G_X' = W_f^T G_Y (rows k, columns j), then col2im scatter-add into
 * dX [H][W][Ci][N].  sabs accumulates |.| of every product the same way. */
int orc_conv_dgrad(const orc_conv* cv, const double* w, const double* dy, double* dx, double* sabs) {
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = out_h(cv) * out_w(cv) * cv->n;
  int64_t Co = cv->c_out;
  int64_t nx = (int64_t)cv->h * cv->w * cv->c_in * cv->n;
  double* wf = build_wf(cv, w);
  double* gyt = (double*)malloc(sizeof(double) * (size_t)(J * Co)); /* gyt[j][co] */
  double* gx = (double*)malloc(sizeof(double) * (size_t)(J * K));   /* G_X'[k][j] as [j][k] */
  double* gs = (double*)malloc(sizeof(double) * (size_t)(J * K));
  if (!wf || !gyt || !gx || !gs) { free(wf); free(gyt); free(gx); free(gs); return -1; }
  for (int64_t j = 0; j < J; ++j) {
    int64_t n = j % cv->n, pos = j / cv->n;
    for (int64_t co = 0; co < Co; ++co) gyt[j * Co + co] = dy[(pos * Co + co) * cv->n + n];
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < J; ++j)
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0, sa = 0.0;
      for (int64_t co = 0; co < Co; ++co) {
        double p = wf[co * K + k] * gyt[j * Co + co];
        acc += p;
        sa += fabs(p);
      }
      gx[j * K + k] = acc;
      gs[j * K + k] = sa;
    }
  /* col2im: each entry of G_X' goes back to the activation it was copied from */
  for (int64_t i = 0; i < nx; ++i) { dx[i] = 0.0; sabs[i] = 0.0; }
  for (int64_t j = 0; j < J; ++j)
    for (int64_t k = 0; k < K; ++k) {
      int64_t s = orc_im2col_src(cv, k, j);
      if (s < 0) continue;
      dx[s] += gx[j * K + k];
      sabs[s] += gs[j * K + k];
    }
  free(wf);
  free(gyt);
  free(gx);
  free(gs);
  return 0;
}

/* G_W = G_Y X'^T (rows co, columns k), reordered to OIHW. */
int orc_conv_wgrad(const orc_conv* cv, const double* dy, const double* x, double* dw, double* sabs) {
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = out_h(cv) * out_w(cv) * cv->n;
  int64_t Co = cv->c_out;
  double* xt = build_im2col_cols(cv, x); /* [j][k] */
  double* gy = (double*)malloc(sizeof(double) * (size_t)(Co * J)); /* [co][j] */
  double* xr = (double*)malloc(sizeof(double) * (size_t)(K * J));  /* X'[k][j] */
  if (!xt || !gy || !xr) { free(xt); free(gy); free(xr); return -1; }
  for (int64_t j = 0; j < J; ++j) {
    int64_t n = j % cv->n, pos = j / cv->n;
    for (int64_t co = 0; co < Co; ++co) gy[co * J + j] = dy[(pos * Co + co) * cv->n + n];
    for (int64_t k = 0; k < K; ++k) xr[k * J + j] = xt[j * K + k];
  }
  free(xt);
#pragma omp parallel for schedule(static)
  for (int64_t co = 0; co < Co; ++co)
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0.0, sa = 0.0;
      for (int64_t j = 0; j < J; ++j) {
        double p = gy[co * J + j] * xr[k * J + j];
        acc += p;
        sa += fabs(p);
      }
      int64_t ci = k % cv->c_in, tap = k / cv->c_in;
      int64_t kw = tap % cv->k_w, kh = tap / cv->k_w;
      int64_t o = ((co * cv->c_in + ci) * cv->k_h + kh) * cv->k_w + kw;
      dw[o] = acc;
      sabs[o] = sa;
    }
  free(gy);
  free(xr);
  return 0;
}

/* ---- the same three definitions evaluated one output at a time, for        */
/* sampled checks of shapes whose explicit im2col would not fit in memory.     */

int orc_conv_fwd_points(const orc_conv* cv, const double* w, const double* x, const int64_t* idx,
                        int64_t npts, double* val, double* sabs) {
  int64_t Ho = out_h(cv), Wo = out_w(cv);
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < npts; ++t) {
    int64_t o = idx[t];
    int64_t n = o % cv->n, r = o / cv->n;
    int64_t co = r % cv->c_out, pos = r / cv->c_out;
    int64_t j = pos * cv->n + n;
    double acc = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      int64_t s = orc_im2col_src(cv, k, j);
      if (s < 0) continue;
      int64_t ci = k % cv->c_in, tap = k / cv->c_in;
      int64_t kw = tap % cv->k_w, kh = tap / cv->k_w;
      double p = w[((co * cv->c_in + ci) * cv->k_h + kh) * cv->k_w + kw] * x[s];
      acc += p;
      sa += fabs(p);
    }
    (void)Ho; (void)Wo;
    val[t] = acc;
    sabs[t] = sa;
  }
  return 0;
}

int orc_conv_dgrad_points(const orc_conv* cv, const double* w, const double* dy, const int64_t* idx,
                          int64_t npts, double* val, double* sabs) {
  int64_t Ho = out_h(cv), Wo = out_w(cv);
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = Ho * Wo * cv->n;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < npts; ++t) {
    int64_t o = idx[t]; /* in [H][W][Ci][N] */
    int64_t n = o % cv->n, r = o / cv->n;
    int64_t ci = r % cv->c_in, pos = r / cv->c_in;
    int64_t ww = pos % cv->w, hh = pos / cv->w;
    double acc = 0.0, sa = 0.0;
    /* every (k, j) of G_X' that col2im maps onto this activation */
    for (int64_t kh = 0; kh < cv->k_h; ++kh)
      for (int64_t kw = 0; kw < cv->k_w; ++kw) {
        int64_t th = hh + cv->pad_h - kh, tw = ww + cv->pad_w - kw;
        if (th < 0 || tw < 0 || th % cv->stride_h || tw % cv->stride_w) continue;
        int64_t ho = th / cv->stride_h, wo = tw / cv->stride_w;
        if (ho >= Ho || wo >= Wo) continue;
        int64_t j = (ho * Wo + wo) * cv->n + n;
        int64_t k = (kh * cv->k_w + kw) * cv->c_in + ci;
        if (orc_im2col_src(cv, k, j) != o) continue; /* consistency with im2col */
        for (int64_t co = 0; co < cv->c_out; ++co) {
          double p = w[((co * cv->c_in + ci) * cv->k_h + kh) * cv->k_w + kw] *
                     dy[((ho * Wo + wo) * cv->c_out + co) * cv->n + n];
          acc += p;
          sa += fabs(p);
        }
      }
    (void)J; (void)K;
    val[t] = acc;
    sabs[t] = sa;
  }
  return 0;
}

int orc_conv_wgrad_points(const orc_conv* cv, const double* dy, const double* x, const int64_t* idx,
                          int64_t npts, double* val, double* sabs) {
  int64_t Ho = out_h(cv), Wo = out_w(cv);
  int64_t J = Ho * Wo * cv->n;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < npts; ++t) {
    int64_t o = idx[t]; /* OIHW */
    int64_t kw = o % cv->k_w, r = o / cv->k_w;
    int64_t kh = r % cv->k_h;
    r /= cv->k_h;
    int64_t ci = r % cv->c_in, co = r / cv->c_in;
    int64_t k = (kh * cv->k_w + kw) * cv->c_in + ci;
    double acc = 0.0, sa = 0.0;
    for (int64_t j = 0; j < J; ++j) {
      int64_t s = orc_im2col_src(cv, k, j);
      if (s < 0) continue;
      int64_t n = j % cv->n, pos = j / cv->n;
      double p = dy[(pos * cv->c_out + co) * cv->n + n] * x[s];
      acc += p;
      sa += fabs(p);
    }
    val[t] = acc;
    sabs[t] = sa;
  }
  return 0;
}

/* Seven-loop direct convolution (cross-correlation with zero padding) on
 * [H][W][Ci][N] activations and OIHW weights -> [Ho][Wo][Co][N]; an
 * independent definition that the im2col GEMM must match. */
int orc_conv_direct(const orc_conv* cv, const double* w, const double* x, double* y) {
  int64_t Ho = out_h(cv), Wo = out_w(cv);
  for (int64_t n = 0; n < cv->n; ++n)
    for (int64_t co = 0; co < cv->c_out; ++co)
      for (int64_t ho = 0; ho < Ho; ++ho)
        for (int64_t wo = 0; wo < Wo; ++wo) {
          double acc = 0.0;
          for (int64_t ci = 0; ci < cv->c_in; ++ci)
            for (int64_t kh = 0; kh < cv->k_h; ++kh)
              for (int64_t kw = 0; kw < cv->k_w; ++kw) {
                int64_t hh = ho * cv->stride_h - cv->pad_h + kh;
                int64_t ww = wo * cv->stride_w - cv->pad_w + kw;
                if (hh < 0 || hh >= cv->h || ww < 0 || ww >= cv->w) continue;
                acc += w[((co * cv->c_in + ci) * cv->k_h + kh) * cv->k_w + kw] *
                       x[((hh * cv->w + ww) * cv->c_in + ci) * cv->n + n];
              }
          y[((ho * Wo + wo) * cv->c_out + co) * cv->n + n] = acc;
        }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Quantization-event counting for the three flows of Table I (§IV-C).         */
/*   flow 0  MicroQonv: X quantized once before im2col                          */
/*   flow 1  quantize-after-im2col (square 8x8 blocks over X', the extension    */
/*           of Cuyckens et al. to convolution)                                 */
/*   flow 2  DaCapo: X' quantized in 64-element lines, once along the rows for */
/*           the forward GEMM and once along the columns for the backward one   */
/* counts[e] = number of quantizations applied to (copies of) activation e;     */
/* returns the total number of quantization events including the zero-padding  */
/* entries of X'.                                                               */
/* ------------------------------------------------------------------------ */
int64_t orc_count_act_quant(const orc_conv* cv, int flow, int32_t* counts) {
  int64_t nx = (int64_t)cv->h * cv->w * cv->c_in * cv->n;
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = out_h(cv) * out_w(cv) * cv->n;
  for (int64_t i = 0; i < nx; ++i) counts[i] = 0;
  if (flow == 0) {
    for (int64_t i = 0; i < nx; ++i) counts[i] += 1;
    return nx;
  }
  int passes = (flow == 1) ? 1 : 2;
  int64_t events = 0;
  for (int p = 0; p < passes; ++p) {
    /* every entry of X' belongs to exactly one block of the pass's tiling and
     * is quantized once with it */
    for (int64_t k = 0; k < K; ++k)
      for (int64_t j = 0; j < J; ++j) {
        int64_t s = orc_im2col_src(cv, k, j);
        events += 1;
        if (s >= 0) counts[s] += 1;
      }
  }
  return events;
}

/* The same count for the weight (tensor 1) and the output gradient (tensor  */
/* 2), in one training step of the three GEMMs (§II-A, §IV-B):                 */
/*   W  is the A operand of the forward GEMM, whose K runs along C_in, and of  */
/*      the data-gradient GEMM, whose K runs along C_out;                       */
/*   dY is the B operand of the data-gradient GEMM (K along C_out) and the A    */
/*      operand of the weight-gradient GEMM (K along the output positions and   */
/*      the batch).                                                             */
/* A GEMM reads its operands in blocks that lie along its K.  A square 8x8      */
/* block (MicroQonv, flow 0, and the square-block flow 1) lies along both       */
/* dimensions, so one quantization serves both GEMMs; a 64-element line         */
/* (DaCapo, flow 2) lies along one, so each K direction takes a quantization   */
/* of its own (§IV-C).  The tensor is viewed per tap as a rows x cols matrix:   */
/* W as [C_out][C_in] at each of the Kh*Kw taps, dY as [C_out][Ho*Wo*N];       */
/* counts[(tap * rows + r) * cols + c] receives the quantizations of that       */
/* element.  Returns the total number of quantization events, -1 on a bad      */
/* argument.                                                                   */
int64_t orc_count_operand_quant(const orc_conv* cv, int flow, int tensor, int32_t* counts) {
  int64_t taps, rows, cols;
  int kdir[2]; /* K direction of the two GEMMs that read the tensor: 0 rows, 1 cols */
  if (tensor == 1) {
    taps = (int64_t)cv->k_h * cv->k_w; rows = cv->c_out; cols = cv->c_in;
    kdir[0] = 1; /* forward: K = C_in */
    kdir[1] = 0; /* data gradient: K = C_out */
  } else if (tensor == 2) {
    taps = 1; rows = cv->c_out; cols = out_h(cv) * out_w(cv) * cv->n;
    kdir[0] = 0; /* data gradient: K = C_out */
    kdir[1] = 1; /* weight gradient: K = (ho, wo, n) */
  } else {
    return -1;
  }
  if (flow < 0 || flow > 2) return -1;
  for (int64_t i = 0; i < taps * rows * cols; ++i) counts[i] = 0;
  /* the block shapes (br x bc) the flow quantizes the tensor in, one per K
   * direction, a shape that serves several GEMMs quantized once */
  int64_t shapes[2][2];
  int nshapes = 0;
  for (int u = 0; u < 2; ++u) {
    int64_t br = 8, bc = 8;
    if (flow == 2) {
      br = kdir[u] == 0 ? 64 : 1;
      bc = kdir[u] == 1 ? 64 : 1;
    }
    int dup = 0;
    for (int v = 0; v < nshapes; ++v) dup |= shapes[v][0] == br && shapes[v][1] == bc;
    if (!dup) {
      shapes[nshapes][0] = br;
      shapes[nshapes][1] = bc;
      ++nshapes;
    }
  }
  int64_t events = 0;
  for (int v = 0; v < nshapes; ++v) {
    int64_t br = shapes[v][0], bc = shapes[v][1];
    /* every block of the tiling (the last ones cut at the tensor's edge) is
     * quantized once; each of its elements is counted */
    for (int64_t t = 0; t < taps; ++t)
      for (int64_t r0 = 0; r0 < rows; r0 += br)
        for (int64_t c0 = 0; c0 < cols; c0 += bc)
          for (int64_t r = r0; r < r0 + br && r < rows; ++r)
            for (int64_t c = c0; c < c0 + bc && c < cols; ++c) {
              counts[(t * rows + r) * cols + c] += 1;
              events += 1;
            }
  }
  return events;
}

/* Square-block quantization of the explicit quantize-after-im2col matrix
 * (flow 1).  That flow works on the conventional im2col of §II-C, whose rows
 * are the channel-major flattened kernel positions (ci, kh, kw) and whose
 * columns are the sliding windows of each sample in turn (n, ho, wo); the
 * matrix is tiled in 8x8 blocks (K and J multiples of 8).  For each entry
 * (row k, column j of THAT matrix) it returns the code, the block scale and
 * the referenced activation index (-1 for padding), so that the codes given
 * to the several copies of one activation can be compared. */
int orc_quantize_after_im2col(const orc_conv* cv, int fmt, const float* x, uint8_t* xq_codes,
                              uint8_t* xq_scales, int64_t* xq_src, float* t_out) {
  orc_fmt_t f;
  if (fmt_desc(fmt, &f)) return -1;
  int64_t Ho = out_h(cv), Wo = out_w(cv);
  int64_t K = (int64_t)cv->k_h * cv->k_w * cv->c_in;
  int64_t J = Ho * Wo * cv->n;
  if (K % 8 || J % 8) return -1;
  float* xp = (float*)malloc(sizeof(float) * (size_t)(K * J));
  if (!xp) return -1;
  for (int64_t k = 0; k < K; ++k) {
    int64_t kw = k % cv->k_w, t = k / cv->k_w;
    int64_t kh = t % cv->k_h, ci = t / cv->k_h;
    for (int64_t j = 0; j < J; ++j) {
      int64_t wo = j % Wo, t2 = j / Wo;
      int64_t ho = t2 % Ho, n = t2 / Ho;
      /* same entry in the CBF ordering used everywhere else */
      int64_t kc = (kh * cv->k_w + kw) * cv->c_in + ci;
      int64_t jc = (ho * Wo + wo) * cv->n + n;
      int64_t s = orc_im2col_src(cv, kc, jc);
      xq_src[k * J + j] = s;
      xp[k * J + j] = s < 0 ? 0.0f : x[s];
    }
  }
  /* X' viewed as a (K/8) x (J/8) grid of 8x8 blocks: use the activation
   * quantizer on the [1][1][K][J] "tensor" whose blocks are exactly these */
  int64_t nel = K * J;
  uint8_t* codes = (uint8_t*)malloc((size_t)nel);
  uint8_t* scales = (uint8_t*)malloc((size_t)(nel / 64));
  float amax;
  if (!codes || !scales) { free(xp); free(codes); free(scales); return -1; }
  int rc = orc_quantize(ORC_ACT, fmt, ORC_RNE, 0, xp, 1, 1, K, J, NULL, codes, scales, t_out, &amax);
  if (rc == 0) {
    int64_t nbj = J / 8;
    for (int64_t k = 0; k < K; ++k)
      for (int64_t j = 0; j < J; ++j) {
        int64_t b = (k / 8) * nbj + j / 8;
        xq_codes[k * J + j] = codes[b * 64 + (k % 8) * 8 + (j % 8)];
        xq_scales[k * J + j] = scales[b];
      }
  }
  free(xp);
  free(codes);
  free(scales);
  return rc;
}

/* Threads the OpenMP loops above run on (for reporting only). */
int orc_threads(void) { return omp_get_max_threads(); }

/* Sets the threads of the OpenMP loops (timing only: the results do not
   depend on it, every loop writes disjoint outputs). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
