// Implicit-im2col convolution GEMMs on microscaled operands (gfx950 MFMA).
//
// MicroQonv (arXiv 2609.28358, §IV-B) writes the three training GEMMs of a
// convolution on channel-batch-first matrices:
//   forward  Y[co, (ho,wo,n)]      = sum_{(kh,kw,ci)} W[co, (kh,kw,ci)] X'[(kh,kw,ci), (ho,wo,n)]
//   data     dX = col2im(W^T dY)   (gather form below: no dX' in memory)
//   weight   dW[co, (kh,kw,ci)]    = sum_{(ho,wo,n)}  dY[co, (ho,wo,n)] X'[(kh,kw,ci), (ho,wo,n)]
// with X' the im2col of the quantized activation.  Every 8x8 block of every
// operand is one quantization block of its tensor (a (C,N) block of X or dY
// at one position, a (Cout,Cin) block of W at one tap), so an operand tile is
// assembled from whole quantized blocks: X' is never materialized, each block
// is fetched straight from the quantized tensor (32/48/64 bytes + 1 scale
// byte) by the workgroup that needs it.
//
// Exactness: a dequantized element g*B (element value times E4M3 block scale)
// has at most 8 significant bits and an exponent within bf16 range for all
// three element formats, so it is exactly a bf16; a bf16 x bf16 product is
// exact in fp32.  The MFMA therefore sums exact products of the Eq. 7
// factorization (§III-B) and the per-tensor scales T_a * T_b are applied once
// in the epilogue.  Block scales change every 8 elements along K, which the
// E8M0-per-32 scaled MFMA of gfx950 cannot express, hence bf16 MFMA.
//
// Kernel shape: 2 or 4 wave64, tile MT x NT, K stage of KB k-blocks (8 K
// values each) sized so that every thread stages one quantized block per
// stage: small tiles take long stages, so the latency-bound K loop of a
// small layer has few steps.  Two LDS stages.  Each thread fetches its
// block two stages ahead, decodes it and writes its eight 8-value K-lines
// to LDS as 16-byte rows [line][k] (k contiguous), which is exactly the
// operand layout of v_mfma_f32_32x32x16_{f16,bf16} (lane l: row/col l%32,
// K slots 8*(l/32)..+7).
#include <type_traits>
#include <utility>

#include "internal.h"
#include "mx_formats.h"

namespace mx {
namespace {

// LDS layout of a staged tile: lines of KT = 8*KB K values, KB the k-blocks
// of one stage, at a stride of KT + 8 16-bit elements (LS), and logical line
// L stored at physical line L ^ ((L >> 2) & 4) (the two halves of every
// second 8-line block swapped).  The stride is an odd number of 16-byte bank
// quads modulo the 64 banks, so the 16-byte fragment reads of 16 consecutive
// lines hit 16 distinct quads; the swizzle spreads the line writes of
// neighbouring blocks (with KB = 4 they hit the four bank quarters).
template <int KB> struct Lds {
  static constexpr int KT = 8 * KB;
  static constexpr int LS = KT + 8;
  static __device__ __forceinline__ int line(int l) { return (l ^ ((l >> 2) & 4)) * LS; }
};

enum { OP_FWD = 0, OP_DGRAD = 1, OP_WGRAD = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned int u32x6 __attribute__((ext_vector_type(6)));

struct ConvParams {
  int32_t n, c_in, c_out, h, w, k_h, k_w, sh, sw, ph, pw, ho, wo;
  int32_t nb;         // n / 8
  int32_t M;          // GEMM rows
  int32_t ncb;        // column blocks (8 columns each) of the launch's column space
  int32_t kb_total;   // k-blocks (8 each) along K
  int32_t ks_split;   // K steps (of the kernel's KB k-blocks) per split (wgrad)
  int32_t ncol;       // wgrad: columns of one partial (Kh*Kw*Cin)
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_t;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_t;
  float* out;
  uint32_t* amax_out;  // fwd: per-wave max |y| slots (slot 1 + global wave index; nullptr: not wanted)
};

// MFMA operand type: E2M1 and E2M3 blocks decode exactly to fp16 (g*B lies in
// [2^-12, 3360] with at most 8 significant bits); E4M3 x E4M3 spans 2^-18 ..
// 2*10^5, beyond fp16's normal range, and decodes exactly to bf16.
template <int FMT> struct OperandType { static constexpr bool F16 = (FMT != FMT_E4M3); };

// Exponent-only scaling plus mantissa factor of an E4M3 block scale B: the
// gfx950 scaled conversions multiply by 2^floor(log2 scale) only, so
// convert(code, B) * mB == code * B exactly, mB = B / 2^floor(log2 B) (a
// value 1 + m/8).  A zero scale gives mB = 0 (the block decodes to zeros).
struct BlockScale {
  float b;   // B itself, passed as the conversion's scale operand
  float mb;  // mantissa factor
  __device__ __forceinline__ explicit BlockScale(uint32_t code) {
    b = code_value<ScaleFmt>(code);
    mb = (code == 0u) ? 0.0f : __uint_as_float((__float_as_uint(b) & 0x007FFFFFu) | 0x3F800000u);
  }
};

// Raw codes of one block held in registers between the global load and the
// LDS store.  The loads are unconditional: a block outside the tensor (zero
// padding, tails) reads block 0 of the tensor instead and carries mask 0,
// which the decode applies to codes and scale (giving zeros).  Branch-free
// loads keep the wait counts exact, so a fetch stays in flight while the
// intervening K steps compute.
template <int FMT>
struct RawBlock {
  static constexpr int WORDS = block_bytes<FMT>() / 4;
  uint32_t w[WORDS];
  uint32_t scale;
  uint32_t mask;  // ~0 for a block of the tensor, 0 for padding

  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, uint32_t blk, bool ok) {
    const uint64_t b = ok ? blk : 0u;
    const uint4* p = reinterpret_cast<const uint4*>(codes + b * block_bytes<FMT>());
#pragma unroll
    for (int i = 0; i < WORDS / 4; ++i) {
      const uint4 v = p[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
    scale = scales[b];
    mask = ok ? ~0u : 0u;
  }
};

// Staging of one block into LDS, cut into units so that the units can be
// placed between the MFMAs of a K step.  ROWS: unit u (0..7) writes line u =
// block row u.  !ROWS: unit u (0..3) writes lines 2u and 2u+1 = block columns
// 2u, 2u+1 (a 2x2 transpose of the row pairs).  Each unit decodes what it
// writes (E2M3 decodes 32 elements at a time: in the first unit of a 4-row
// group for ROWS, all 64 in unit 0 for !ROWS).
template <int FMT, bool ROWS, int LS>
struct Stager {
  static constexpr int UNITS = ROWS ? 8 : 4;
  BlockScale bs;
  uint32_t mask;
  uint32_t P[8][4];  // pairs (element (r,2j), element (r,2j+1)) as two 16-bit floats
  uint16_t* p_lo;    // lines 0-3 of the block (swizzled halves, see lds_line)
  uint16_t* p_hi;    // lines 4-7

  __device__ __forceinline__ Stager(const RawBlock<FMT>& raw, uint16_t* lo, uint16_t* hi)
      : bs(raw.scale & raw.mask), mask(raw.mask), p_lo(lo), p_hi(hi) {}

  __device__ __forceinline__ uint16_t* line_ptr(int i) const {
    return (i < 4) ? p_lo + i * LS : p_hi + (i - 4) * LS;
  }

  // pair j of row r
  template <int R, int J>
  __device__ __forceinline__ uint32_t pair(const RawBlock<FMT>& raw) const {
    if constexpr (FMT == FMT_E2M1) {
      const _Float16 m = static_cast<_Float16>(bs.mb);
      const f16x2 m2 = {m, m};
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw.w[R] & mask, bs.b, J) * m2);
    } else {
      // exact: at most 7 significant bits, so the bf16 is the high half
      const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.w[2 * R + (J >> 1)] & mask, bs.b, (J & 1) != 0);
      const float lo = f[0] * bs.mb, hi = f[1] * bs.mb;
      return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    }
  }

  // E2M3: rows 4G .. 4G+3 (192 consecutive bits) into P
  template <int G>
  __device__ __forceinline__ void fp6_group(const RawBlock<FMT>& raw) {
    const _Float16 m = static_cast<_Float16>(bs.mb);
    const f16x2 m2 = {m, m};
    u32x6 src;
    src[0] = raw.w[6 * G + 0] & mask; src[1] = raw.w[6 * G + 1] & mask; src[2] = raw.w[6 * G + 2] & mask;
    src[3] = raw.w[6 * G + 3] & mask; src[4] = raw.w[6 * G + 4] & mask; src[5] = raw.w[6 * G + 5] & mask;
    const auto v = __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(src, bs.b);
    struct Words { uint32_t u[16]; };
    const Words wv = __builtin_bit_cast(Words, v);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      P[4 * G + i / 4][i % 4] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, wv.u[i]) * m2);
  }

  template <int U>
  __device__ __forceinline__ void unit(const RawBlock<FMT>& raw) {
    if constexpr (ROWS) {
      if constexpr (FMT == FMT_E2M3) {
        if constexpr (U % 4 == 0) fp6_group<U / 4>(raw);
      } else {
        P[U][0] = pair<U, 0>(raw);
        P[U][1] = pair<U, 1>(raw);
        P[U][2] = pair<U, 2>(raw);
        P[U][3] = pair<U, 3>(raw);
      }
      *reinterpret_cast<uint4*>(line_ptr(U)) = make_uint4(P[U][0], P[U][1], P[U][2], P[U][3]);
    } else {
      if constexpr (FMT == FMT_E2M3) {
        if constexpr (U == 0) {
          fp6_group<0>(raw);
          fp6_group<1>(raw);
        }
      } else {
        P[0][U] = pair<0, U>(raw); P[1][U] = pair<1, U>(raw);
        P[2][U] = pair<2, U>(raw); P[3][U] = pair<3, U>(raw);
        P[4][U] = pair<4, U>(raw); P[5][U] = pair<5, U>(raw);
        P[6][U] = pair<6, U>(raw); P[7][U] = pair<7, U>(raw);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t sel = e ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = __builtin_amdgcn_perm(P[1][U], P[0][U], sel);
        o.y = __builtin_amdgcn_perm(P[3][U], P[2][U], sel);
        o.z = __builtin_amdgcn_perm(P[5][U], P[4][U], sel);
        o.w = __builtin_amdgcn_perm(P[7][U], P[6][U], sel);
        *reinterpret_cast<uint4*>(line_ptr(2 * U + e)) = o;
      }
    }
  }
};

// Division by a runtime constant d >= 1 for dividends below 2^31 (block
// and k-block indices): q = floor(x * m / 2^sh) with sh = 31 + ceil(log2 d)
// and m = ceil(2^sh / d) < 2^32.  The product overshoots x/d by less than
// x / 2^sh < 1/d, which never crosses the next integer, so q is exact.
// Branch-free, so the k-block walk can be scheduled between MFMAs.
struct FastDiv {
  uint32_t m, d;
  int sh;
  __device__ __forceinline__ void init(uint32_t dv) {
    d = dv;
    const int l = dv > 1 ? 32 - __builtin_clz(dv - 1) : 0;
    sh = 31 + l;
    m = static_cast<uint32_t>(((static_cast<uint64_t>(1) << sh) + dv - 1) / dv);
  }
  __device__ __forceinline__ uint32_t div(uint32_t x) const {
    return static_cast<uint32_t>((static_cast<uint64_t>(x) * m) >> sh);
  }
};

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(const uint16_t* pa, const uint16_t* pb, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(pa),
                                                  *reinterpret_cast<const f16x8*>(pb), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(pa),
                                                   *reinterpret_cast<const bf16x8*>(pb), c, 0, 0, 0);
}

// Per-workgroup context shared by the conv kernels: the tile this
// workgroup computes, the data-gradient phase or weight-gradient split of
// the launch's z index, and the quantized block one thread stages per K
// step (thread t < ABLK stages A blocks, the next BBLK threads B blocks).
template <int OP, int MT, int NT, int KB>
struct TileCtx {
  static constexpr int ABLK = (MT / 8) * KB, BBLK = (NT / 8) * KB;
  int bx, by, bz, rb0, cb0, cbin, cbout;
  int phh, phw, kh0, kw0, nkh, nkw, hp, wp;
  int kb_begin, kb_end, ncb_launch;
  bool is_a, active, in_range;
  int lblk, kbl, gblk;
  int col_nb, col_cib;
  int sp_y, sp_x, st_y, st_x;
  FastDiv div_inner, div_b;
  uint32_t kb;  // the k-block this thread stages next

  // false: the workgroup has no output (a data-gradient phase smaller than
  // the grid)
  __device__ __forceinline__ bool init(const ConvParams& p, int tid) {
    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2)
    // in launch order.  Renumber them so that every XCD works on one
    // contiguous range of tiles: neighbouring output tiles share most of
    // their quantized input blocks (the im2col halo, and the weight tile).
    {
      const int total = gridDim.x * gridDim.y * gridDim.z;
      const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
      const int q = total >> 3, r = total & 7, xcd = lin & 7, idx = lin >> 3;
      const int nl = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
      bx = nl % gridDim.x;
      const int t = nl / gridDim.x;
      by = t % gridDim.y;
      bz = t / gridDim.y;
    }
    rb0 = by * (MT / 8);
    cb0 = bx * (NT / 8);
    cbin = p.c_in >> 3;
    cbout = p.c_out >> 3;

    // per-launch-z context: data-gradient phase or weight-gradient split
    phh = 0; phw = 0; kh0 = 0; kw0 = 0; nkh = p.k_h; nkw = p.k_w; hp = 0; wp = 0;
    kb_begin = 0;
    kb_end = p.kb_total;
    if constexpr (OP == OP_DGRAD) {
      // output pixels (h, w) with h = phh + sh*h', w = phw + sw*w' receive
      // the taps kh = (phh + ph) mod sh (+ sh, ...), kw likewise
      phh = bz / p.sw;
      phw = bz - phh * p.sw;
      kh0 = (phh + p.ph) % p.sh;
      kw0 = (phw + p.pw) % p.sw;
      nkh = kh0 < p.k_h ? (p.k_h - kh0 + p.sh - 1) / p.sh : 0;
      nkw = kw0 < p.k_w ? (p.k_w - kw0 + p.sw - 1) / p.sw : 0;
      hp = (p.h - phh + p.sh - 1) / p.sh;
      wp = (p.w - phw + p.sw - 1) / p.sw;
      if (cb0 >= hp * wp * p.nb) return false;
      kb_end = nkh * nkw * cbout;
    } else if constexpr (OP == OP_WGRAD) {
      kb_begin = bz * p.ks_split * KB;
      kb_end = min(p.kb_total, kb_begin + p.ks_split * KB);
      if (kb_begin > kb_end) kb_begin = kb_end;
    }
    ncb_launch = (OP == OP_DGRAD) ? hp * wp * p.nb : p.ncb;

    // the block this thread stages every step
    is_a = tid < ABLK;
    const int t_local = is_a ? tid : tid - ABLK;
    active = tid < ABLK + BBLK;
    lblk = t_local / KB;  // line block (8 lines) within the tile
    kbl = active ? t_local - lblk * KB : 0;
    gblk = (is_a ? rb0 : cb0) + lblk;
    in_range = active && (is_a ? (gblk < (p.M >> 3)) : (gblk < ncb_launch));

    // column-block geometry fixed over the K loop
    int col_y = 0, col_x = 0;            // FWD: output (ho, wo); DGRAD: input pixel (h, w)
    int col_kh = 0, col_kw = 0;          // WGRAD: tap
    col_nb = 0;
    col_cib = 0;
    if (!is_a && in_range) {
      if constexpr (OP == OP_FWD) {
        const int pos = gblk / p.nb;
        col_nb = gblk - pos * p.nb;
        col_y = pos / p.wo;
        col_x = pos - col_y * p.wo;
      } else if constexpr (OP == OP_DGRAD) {
        const int pos = gblk / p.nb;
        col_nb = gblk - pos * p.nb;
        const int hq = pos / wp;
        col_y = phh + p.sh * hq;
        col_x = phw + p.sw * (pos - hq * wp);
      } else {
        const int tap = gblk / cbin;
        col_cib = gblk - tap * cbin;
        col_kh = tap / p.k_w;
        col_kw = tap - col_kh * p.k_w;
      }
    }

    // The k-blocks one thread stages are kb, kb+KB, ...; each is split as
    //   FWD  : kb = tap * CBin + cib,  tap = kh * Kw + kw          (a = kh, b = kw)
    //   DGRAD: kb = ti * CBout + cob,  ti over the phase's valid taps (a, b)
    //   WGRAD: kb = pos * NB + nbk,    pos = ho * Wo + wo          (a = ho, b = wo)
    if constexpr (OP == OP_FWD) { div_inner.init(cbin); div_b.init(p.k_w); }
    else if constexpr (OP == OP_DGRAD) { div_inner.init(cbout); div_b.init(nkw > 0 ? nkw : 1); }
    else { div_inner.init(p.nb); div_b.init(p.wo); }
    kb = static_cast<uint32_t>(kb_begin + kbl);
    // offsets of the spatial gather: the source position of a tap (a, b) is
    // (sp_y + a * st_y, sp_x + b * st_x)
    sp_y = 0; sp_x = 0; st_y = 1; st_x = 1;
    if constexpr (OP == OP_FWD) {
      sp_y = col_y * p.sh - p.ph; sp_x = col_x * p.sw - p.pw;
    } else if constexpr (OP == OP_DGRAD) {
      // dY row of the tap: (col_y + ph - kh) / sh with kh = kh0 + sh * a,
      // an exact division by construction of the phase
      sp_y = (col_y + p.ph - kh0) / p.sh; sp_x = (col_x + p.pw - kw0) / p.sw;
      st_y = -1; st_x = -1;
    } else {
      sp_y = col_kh - p.ph; sp_x = col_kw - p.pw; st_y = p.sh; st_x = p.sw;
    }
    return true;
  }

  // The quantized block of this thread's slot at k-block kb, and whether it
  // exists (false in the zero padding or outside the GEMM).  Straight-line
  // 32-bit arithmetic: indices past the tensor are computed but never used.
  __device__ __forceinline__ bool locate(const ConvParams& p, uint32_t& blk) const {
    const uint32_t outer = div_inner.div(kb);
    const uint32_t inner = kb - outer * div_inner.d;
    const uint32_t a = div_b.div(outer);
    const uint32_t b = outer - a * div_b.d;
    const int y = sp_y + static_cast<int>(a) * st_y, x = sp_x + static_cast<int>(b) * st_x;
    uint32_t ba, bb;
    bool inb;
    if constexpr (OP == OP_FWD) {
      ba = ((a * p.k_w + b) * cbout + gblk) * cbin + inner;
      inb = static_cast<uint32_t>(y) < static_cast<uint32_t>(p.h) && static_cast<uint32_t>(x) < static_cast<uint32_t>(p.w);
      bb = ((static_cast<uint32_t>(y) * p.w + x) * cbin + inner) * p.nb + col_nb;
    } else if constexpr (OP == OP_DGRAD) {
      const uint32_t kh = kh0 + p.sh * a, kwi = kw0 + p.sw * b;
      ba = ((kh * p.k_w + kwi) * cbout + inner) * cbin + gblk;
      inb = static_cast<uint32_t>(y) < static_cast<uint32_t>(p.ho) && static_cast<uint32_t>(x) < static_cast<uint32_t>(p.wo);
      bb = ((static_cast<uint32_t>(y) * p.wo + x) * cbout + inner) * p.nb + col_nb;
    } else {
      ba = ((a * p.wo + b) * cbout + gblk) * p.nb + inner;
      inb = static_cast<uint32_t>(y) < static_cast<uint32_t>(p.h) && static_cast<uint32_t>(x) < static_cast<uint32_t>(p.w);
      bb = ((static_cast<uint32_t>(y) * p.w + x) * cbin + col_cib) * p.nb + inner;
    }
    blk = is_a ? ba : bb;
    return in_range && kb < static_cast<uint32_t>(kb_end) && (is_a || inb);
  }
};

// Epilogue: D lane layout of the 32x32 MFMA: column lane%32, rows
// 8*(v/4) + 4*(lane/32) + v%4 for accumulator element v.  fwd / dgrad write
// the scaled outputs in place; wgrad writes unscaled split partials.
template <int OP, int MT, int NT, int KB, int WTM, int WTN, int RM, int RN>
__device__ __forceinline__ void store_tile(const ConvParams& p, const TileCtx<OP, MT, NT, KB>& t,
                                           const f32x16 (&acc)[RM][RN], int lane, int wm, int wn) {
  float scale = 1.0f;
  if constexpr (OP != OP_WGRAD) scale = (*p.a_t) * (*p.b_t);
  int64_t row_stride;
  if constexpr (OP == OP_WGRAD) row_stride = p.ncol;
  else row_stride = p.n;

  uint32_t ymax = 0;  // fwd: max over the written outputs of their sign-cleared bits
  auto put = [&](float* q, float v) {
    *q = v;
    if constexpr (OP == OP_FWD) ymax = max(ymax, __float_as_uint(v) & 0x7FFFFFFFu);
  };
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int col = t.cb0 * 8 + wn * WTN + j * 32 + (lane & 31);  // column in the launch space
    const int cbk = col >> 3, c = col & 7;
    if (cbk >= t.ncb_launch) continue;
    int64_t colbase;
    if constexpr (OP == OP_FWD) {
      const int pos = cbk / p.nb, nbk = cbk - pos * p.nb;
      colbase = static_cast<int64_t>(pos) * p.c_out * p.n + nbk * 8 + c;
    } else if constexpr (OP == OP_DGRAD) {
      const int pos = cbk / p.nb, nbk = cbk - pos * p.nb;
      const int hq = pos / t.wp;
      const int hh = t.phh + p.sh * hq, ww = t.phw + p.sw * (pos - hq * t.wp);
      colbase = (static_cast<int64_t>(hh) * p.w + ww) * p.c_in * p.n + nbk * 8 + c;
    } else {
      colbase = static_cast<int64_t>(t.bz) * p.M * p.ncol + col;
    }
    float* out = p.out + colbase;
    const int row0 = t.rb0 * 8 + wm * WTM + 4 * (lane >> 5);
    if (t.rb0 * 8 + wm * WTM + WTM <= p.M) {
      // the wave's rows all exist (uniform test): no per-element branch
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          put(out + static_cast<int64_t>(row0 + i * 32 + 8 * (v >> 2) + (v & 3)) * row_stride, acc[i][j][v] * scale);
    } else {
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = row0 + i * 32 + 8 * (v >> 2) + (v & 3);
          if (row < p.M) put(out + static_cast<int64_t>(row) * row_stride, acc[i][j][v] * scale);
        }
    }
  }
  if constexpr (OP == OP_FWD) {
    // producer-fused amax: every wave stores the max of its outputs in its
    // own slot (no atomics); k_amax_finish reduces the slots.  The uint order
    // of sign-cleared bits is the order of |y|, NaN above everything, as in
    // the quantizer's amax pass.
    if (p.amax_out != nullptr) {
      for (int off = 32; off > 0; off >>= 1)
        ymax = max(ymax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(ymax), off)));
      const int64_t wg = blockIdx.x + static_cast<int64_t>(gridDim.x) * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
      if (lane == 0) p.amax_out[1 + wg * (blockDim.x >> 6) + (threadIdx.x >> 6)] = ymax;
    }
  }
}

template <int OP, int FMT, int MT, int NT, int WM, int WAVES, int KB>
__global__ __launch_bounds__(WAVES * 64) void k_conv(const ConvParams p) {
  constexpr int WN = WAVES / WM;
  constexpr int WTM = MT / WM, WTN = NT / WN;
  constexpr int RM = WTM / 32, RN = WTN / 32;
  constexpr int ABLK = (MT / 8) * KB, BBLK = (NT / 8) * KB;
  constexpr int NK = KB / 2;  // 16-wide MFMA K slices per stage
  constexpr int LS = Lds<KB>::LS;
  static_assert(KB % 2 == 0, "a stage is a whole number of 16-wide K slices");
  constexpr bool F16 = OperandType<FMT>::F16;
  static_assert(ABLK + BBLK <= WAVES * 64, "one block per thread per stage");
  static_assert(RM >= 1 && RN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile of 32x32 MFMAs");

  // NSTAGE stages of MT + NT lines, plus 8 lines that threads without a
  // block write their zeros into (keeps the staging code branch-free).  The
  // 256x256 tile runs one workgroup per CU and takes three stages; the
  // smaller tiles keep two, so that two workgroups fit on a CU.
  constexpr int NSTAGE = (MT == 256) ? 3 : 2;
  constexpr int STAGE = (MT + NT + 8) * LS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[NSTAGE][STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx<OP, MT, NT, KB> t;
  if (!t.init(p, tid)) return;
  const bool is_a = t.is_a;
  const int line = !t.active ? MT + NT : is_a ? t.lblk * 8 : MT + t.lblk * 8;
  // swizzled addresses of the block's two line halves (see Lds)
  const int rot = (line >> 2) & 4;
  const int lo_off = (line + rot) * LS + t.kbl * 8;
  const int hi_off = (line + (rot ^ 4)) * LS + t.kbl * 8;
  const int kb_begin = t.kb_begin, kb_end = t.kb_end;

  // A lines are block rows for FWD (co rows, ci along K) and WGRAD (co rows,
  // n along K), block columns for DGRAD (ci lines, co along K).  B lines are
  // block columns for FWD (n lines, ci along K) and DGRAD (n lines, co along
  // K), block rows for WGRAD (ci lines, n along K).
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);

  // Two register sets of raw codes: the global loads of a block are issued
  // two K steps before its decode, so their latency hides behind two rounds
  // of MFMAs.
  RawBlock<FMT> raw0, raw1;
  const uint8_t* my_codes = is_a ? p.a_codes : p.b_codes;
  const uint8_t* my_scales = is_a ? p.a_scales : p.b_scales;
  auto fetch = [&](RawBlock<FMT>& raw) {
    uint32_t blk = 0;
    const bool ok = t.locate(p, blk);
    raw.load(my_codes, my_scales, blk, ok);
    t.kb += KB;
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // per-lane LDS offsets of the MFMA fragments (row / column lane%32 of each
  // 32-wide sub-tile; the two K halves of a 16-wide slice are 8 apart)
  int a_off[RM], b_off[RN];
#pragma unroll
  for (int i = 0; i < RM; ++i) a_off[i] = Lds<KB>::line(wm * WTM + i * 32 + (lane & 31)) + (lane >> 5) * 8;
#pragma unroll
  for (int j = 0; j < RN; ++j) b_off[j] = Lds<KB>::line(MT + wn * WTN + j * 32 + (lane & 31)) + (lane >> 5) * 8;

  // One K step on stage `cur` is NK slices of 16 K values.  Fragments are
  // double-buffered in registers: the LDS reads of slice k+1 are issued
  // before the MFMAs of slice k.  The staging units of a future block (`nxt`,
  // into stage `dst`) are spread between the MFMAs.
  //   2 stages: dst is the next step's stage; the staging units sit in
  //     slices 0..NK-2, then the workgroup barrier, after which the first
  //     slice of the next stage is read while the last slice's MFMAs run.
  //   3 stages: dst is the stage two steps ahead, so the next stage is
  //     already complete: its first slice is read during the last slice and
  //     the barrier closes the step; the staging units spread over (nearly)
  //     all MFMAs of the step, keeping the VALU work per MFMA within what
  //     one wave hides behind a 32-cycle MFMA.
  // An MFMA must never sit inside a branch that diverges within a wave (the
  // wave would execute both sides).  When the A/B staging split falls on wave
  // boundaries (ABLK a multiple of 64) the branch on is_a is wave-uniform and
  // each side carries the MFMA sequence with its own staging units;
  // otherwise one MFMA sequence carries both kinds of units, predicated.
  constexpr int NMF_ALL = (NSTAGE == 3 ? NK : NK - 1) * RM * RN;
  // MFMAs that carry staging units: the first 7/8 (3 stages) or 3/4 (2
  // stages) of those, so that the LDS writes have landed when the barrier
  // comes
  constexpr int NMF = NSTAGE == 3 ? (NMF_ALL * 7 + 7) / 8 : (NMF_ALL * 3 + 3) / 4;
  using StA = Stager<FMT, A_ROWS, LS>;
  using StB = Stager<FMT, B_ROWS, LS>;
  typedef __attribute__((__vector_size__(8 * sizeof(uint16_t)))) uint16_t u16x8;
  u16x8 fa0[RM], fb0[RN], fa1[RM], fb1[RN];
  auto read_slice = [&](int stage, int kk, u16x8 (&fa)[RM], u16x8 (&fb)[RN]) {
    const uint16_t* base = lds[stage] + kk * 16;
#pragma unroll
    for (int i = 0; i < RM; ++i) fa[i] = *reinterpret_cast<const u16x8*>(base + a_off[i]);
#pragma unroll
    for (int j = 0; j < RN; ++j) fb[j] = *reinterpret_cast<const u16x8*>(base + b_off[j]);
  };
  // staging units due after MFMA m (m < NMF): unit u of NU follows MFMA
  // ceil((u+1) * NMF / NU) - 1 (several per MFMA when NU > NMF).  Each MFMA
  // with the work placed after it is closed by a scheduling barrier, so the
  // compiler keeps this interleave instead of clumping the VALU work.
  auto units_after = [&](auto& st, const RawBlock<FMT>& nxt, int m, bool on) {
    using St = std::remove_reference_t<decltype(st)>;
    [&]<int... U>(std::integer_sequence<int, U...>) {
      ((((U + 1) * NMF + St::UNITS - 1) / St::UNITS - 1 == m && on ? (st.template unit<U>(nxt), 0) : 0), ...);
    }(std::make_integer_sequence<int, St::UNITS>());
  };
  // slice KK of a step on stage cur whose slice 0 sits in fragment set PAR;
  // `nstage` is the stage of the next step
  auto slice = [&]<int PAR, int KK>(int cur, int nstage, auto&& after) {
    constexpr int CUR = (PAR + KK) & 1;
    auto& fa_c = CUR ? fa1 : fa0;
    auto& fb_c = CUR ? fb1 : fb0;
    auto& fa_n = CUR ? fa0 : fa1;
    auto& fb_n = CUR ? fb0 : fb1;
    constexpr bool CARRIES = NSTAGE == 3 || KK + 1 < NK;  // staging units in this slice
    if constexpr (KK + 1 < NK) {
      read_slice(cur, KK + 1, fa_n, fb_n);
    } else {
      if constexpr (NSTAGE == 2) __syncthreads();  // next stage complete; cur no longer read
      read_slice(nstage, 0, fa_n, fb_n);
    }
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) {
        acc[i][j] = mfma32<F16>(reinterpret_cast<const uint16_t*>(&fa_c[i]),
                                reinterpret_cast<const uint16_t*>(&fb_c[j]), acc[i][j]);
        if constexpr (CARRIES) after((KK * RM + i) * RN + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    if constexpr (NSTAGE == 3 && KK + 1 == NK) __syncthreads();  // dst complete; cur free
  };
  auto mma_step = [&]<int PAR>(int cur, int nstage, auto&& after) {
    [&]<int... KK>(std::integer_sequence<int, KK...>) {
      (slice.template operator()<PAR, KK>(cur, nstage, after), ...);
    }(std::make_integer_sequence<int, NK>());
  };
  // One step: MFMAs on stage cur; stage `nxt` into stage dst; the global
  // loads of a later step go into `fut` right after the first MFMA.
  auto run_step = [&]<int PAR>(int cur, int nstage, int dst, const RawBlock<FMT>& nxt, RawBlock<FMT>& fut) {
    uint16_t* lo = &lds[dst][lo_off];
    uint16_t* hi = &lds[dst][hi_off];
    if constexpr (ABLK % 64 == 0) {
      if (is_a) {
        StA sa(nxt, lo, hi);
        mma_step.template operator()<PAR>(cur, nstage, [&](int m) {
          if (m == 0) fetch(fut);
          units_after(sa, nxt, m, true);
        });
      } else {
        StB sb(nxt, lo, hi);
        mma_step.template operator()<PAR>(cur, nstage, [&](int m) {
          if (m == 0) fetch(fut);
          units_after(sb, nxt, m, true);
        });
      }
    } else {
      StA sa(nxt, lo, hi);
      StB sb(nxt, lo, hi);
      mma_step.template operator()<PAR>(cur, nstage, [&](int m) {
        if (m == 0) fetch(fut);
        units_after(sa, nxt, m, is_a);
        units_after(sb, nxt, m, !is_a);
      });
    }
  };
  auto stage_all = [&](const RawBlock<FMT>& raw, int stage) {
    if (is_a) {
      StA st(raw, &lds[stage][lo_off], &lds[stage][hi_off]);
      [&]<int... U>(std::integer_sequence<int, U...>) { (st.template unit<U>(raw), ...); }(
          std::make_integer_sequence<int, StA::UNITS>());
    } else {
      StB st(raw, &lds[stage][lo_off], &lds[stage][hi_off]);
      [&]<int... U>(std::integer_sequence<int, U...>) { (st.template unit<U>(raw), ...); }(
          std::make_integer_sequence<int, StB::UNITS>());
    }
  };

  // Steps past the end fetch padding (mask 0) and stage into a stage that
  // is never read again: no branch around a fetch or a staging unit.
  const int nsteps = (kb_end - kb_begin + KB - 1) / KB;
  constexpr int PAR1 = NK & 1;  // fragment set of slice 0 in odd steps
  if (nsteps > 0) {
    if constexpr (NSTAGE == 2) {
      fetch(raw0);
      fetch(raw1);
      stage_all(raw0, 0);
      __syncthreads();
      read_slice(0, 0, fa0, fb0);
      for (int s = 0; s < nsteps; s += 2) {
        // step s reads stage 0; raw1 holds step s+1, raw0 is free
        run_step.template operator()<0>(0, 1, 1, raw1, raw0);
        if (s + 1 >= nsteps) break;
        // step s+1 reads stage 1; raw0 holds step s+2, raw1 is free
        run_step.template operator()<PAR1>(1, 0, 0, raw0, raw1);
      }
    } else {
      // step s computes stage s%3, stages step s+2 (held in raw[s%2]) into
      // stage (s+2)%3 and fetches step s+3 into raw[(s+1)%2]
      fetch(raw0);
      fetch(raw1);
      stage_all(raw0, 0);
      stage_all(raw1, 1);
      fetch(raw0);  // step 2
      __syncthreads();
      read_slice(0, 0, fa0, fb0);
      int cur = 0;
      for (int s = 0; s < nsteps; s += 2) {
        const int c1 = cur == 2 ? 0 : cur + 1, c2 = c1 == 2 ? 0 : c1 + 1;
        run_step.template operator()<0>(cur, c1, c2, raw0, raw1);
        if (s + 1 >= nsteps) break;
        const int c3 = c2 == 2 ? 0 : c2 + 1;
        run_step.template operator()<PAR1>(c1, c2, c3, raw1, raw0);
        cur = c2;
      }
    }
  }

  store_tile<OP, MT, NT, KB, WTM, WTN, RM, RN>(p, t, acc, lane, wm, wn);
}

// ---- E2M1 operands: decode at fragment read ------------------------------
//
// An fp16 stage of the kernel above costs the LDS one 16-byte write and two
// 16-byte reads per 8 K values of a line, which is as much LDS time as the
// MFMAs take on the 256-wide tiles.  For E2M1 the LDS holds the raw 4-bit
// codes instead (4 bytes per line per k-block) and every wave decodes its
// own fragments in registers, between its MFMAs.
//
// Stage layout (KB = 4, one k-quad = two 16-wide K slices):
//   codes  [line][16 B]: the 4 k-blocks of a line in the order 0, 2, 1, 3,
//          so that lane half h reads k-blocks h and 2+h (its K slots in
//          slice 0 and slice 1) with one 8-byte read; the 8 lines of a line
//          block are XOR-permuted by the block index, which keeps the
//          staging writes (one row of 8 codes = 4 bytes each) to at most two
//          per bank while the fragment reads still cover 512 contiguous
//          bytes;
//   scales [line block][16 B]: one word per k-block, same order: the fp32
//          exponent field of B with the fp16 mantissa factor mB in the low
//          16 bits.  The hardware conversion takes only the exponent of its
//          scale operand, so the word serves as the scale directly.

// Transpose an 8x8 matrix of 4-bit codes held as 8 rows of 8 nibbles
// (nibble c of w[r] = element (r, c)): 4x4 blocks, then 2x2, then single
// nibbles.
__device__ __forceinline__ void transpose_nibbles(uint32_t (&w)[8]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t a = w[r], b = w[r + 4];
    w[r] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    w[r + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int r = 0; r < 8; r += (r & 1) ? 3 : 1) {  // r = 0, 1, 4, 5
    const uint32_t a = w[r], b = w[r + 2];
    w[r] = __builtin_amdgcn_perm(b, a, 0x06020400u);
    w[r + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
  }
#pragma unroll
  for (int r = 0; r < 8; r += 2) {
    const uint32_t a = w[r], b = w[r + 1];
    w[r] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    w[r + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// Scale word of an E4M3 block scale code (0 for a zero scale).
__device__ __forceinline__ uint32_t scale_word(uint32_t code) {
  const float b = code_value<ScaleFmt>(code);
  const uint32_t bits = __float_as_uint(b);
  const _Float16 mb = static_cast<_Float16>(__uint_as_float((bits & 0x007FFFFFu) | 0x3F800000u));
  return code == 0u ? 0u : (bits & 0x7F800000u) | __builtin_bit_cast(uint16_t, mb);
}

// Eight exact fp16 values code * B of one fragment: the conversion applies
// 2^exponent(B), the packed multiply the mantissa factor mB.
__device__ __forceinline__ f16x8 decode_frag(uint32_t codes, uint32_t sw) {
  const float sc = __uint_as_float(sw);
  const _Float16 m = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sw & 0xFFFFu));
  const f16x2 m2 = {m, m};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 0) * m2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 1) * m2;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 2) * m2;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 3) * m2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// two workgroups per CU: at most 256 registers per wave
template <int OP, int MT, int NT, int WM, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_conv4(const ConvParams p) {
  constexpr int KB = 4;
  constexpr int WN = WAVES / WM;
  constexpr int WTM = MT / WM, WTN = NT / WN;
  constexpr int RM = WTM / 32, RN = WTN / 32;
  constexpr int ABLK = (MT / 8) * KB, BBLK = (NT / 8) * KB;
  static_assert(ABLK + BBLK <= WAVES * 64, "one block per thread per stage");
  static_assert(ABLK % 64 == 0, "the A/B staging split falls on wave boundaries");
  static_assert(RM >= 1 && RN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile of 32x32 MFMAs");
  constexpr int LINES = MT + NT + 8;  // + 8 spare lines for threads without a block
  constexpr int CODE_B = LINES * 16;
  constexpr int STAGE_B = CODE_B + (LINES / 8) * 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx<OP, MT, NT, KB> t;
  if (!t.init(p, tid)) return;
  const bool is_a = t.is_a;
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);
  const bool rows = is_a ? A_ROWS : B_ROWS;  // uniform per wave

  // staging addresses of this thread's block: row r goes to physical line
  // lb*8 + (r ^ (lb & 7)) at the k-block's slot
  const int lb = !t.active ? (MT + NT) / 8 : is_a ? t.lblk : MT / 8 + t.lblk;
  const int slot = ((t.kbl & 1) << 1) | ((t.kbl >> 1) & 1);
  const int st_code = lb * 8 * 16 + slot * 4;
  const int st_perm = lb & 7;
  const int st_scale = CODE_B + lb * 16 + slot * 4;

  const uint8_t* my_codes = is_a ? p.a_codes : p.b_codes;
  const uint8_t* my_scales = is_a ? p.a_scales : p.b_scales;
  RawBlock<FMT_E2M1> g;
  auto fetch = [&]() {
    uint32_t blk = 0;
    const bool ok = t.locate(p, blk);
    g.load(my_codes, my_scales, blk, ok);
    t.kb += KB;
  };
  // stage the fetched block: its 8 code lines (transposed first when K runs
  // along the block's rows) and its scale word
  auto stage_block = [&](int stg) {
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) w[r] = g.w[r] & g.mask;
    if (!rows) transpose_nibbles(w);
    const uint32_t sw = scale_word(g.scale & g.mask);
    uint8_t* base = lds[stg];
#pragma unroll
    for (int r = 0; r < 8; ++r) *reinterpret_cast<uint32_t*>(base + st_code + ((r ^ st_perm) * 16)) = w[r];
    *reinterpret_cast<uint32_t*>(base + st_scale) = sw;
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment read offsets (physical line of logical line L, lane half h)
  auto pline = [](int L) { return L ^ ((L >> 3) & 7); };
  int a_code[RM], a_scale[RM], b_code[RN], b_scale[RN];
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int L = wm * WTM + i * 32 + (lane & 31);
    a_code[i] = pline(L) * 16 + (lane >> 5) * 8;
    a_scale[i] = CODE_B + (L >> 3) * 16 + (lane >> 5) * 8;
  }
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int L = MT + wn * WTN + j * 32 + (lane & 31);
    b_code[j] = pline(L) * 16 + (lane >> 5) * 8;
    b_scale[j] = CODE_B + (L >> 3) * 16 + (lane >> 5) * 8;
  }
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  // raw fragments of one stage (.x slice 0, .y slice 1)
  u32x2 ra[RM], sa[RM], rb[RN], sbv[RN];
  auto read_raw = [&](int stg) {
    const uint8_t* base = lds[stg];
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      ra[i] = *reinterpret_cast<const u32x2*>(base + a_code[i]);
      sa[i] = *reinterpret_cast<const u32x2*>(base + a_scale[i]);
    }
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      rb[j] = *reinterpret_cast<const u32x2*>(base + b_code[j]);
      sbv[j] = *reinterpret_cast<const u32x2*>(base + b_scale[j]);
    }
  };
  // one slice: the A fragments are decoded up front, each B fragment just
  // before its column of MFMAs.  The scheduling barriers keep this order:
  // left free, the scheduler hoists all decodes to the top and spills.
  auto slice = [&](bool second) {
    f16x8 fa[RM];
#pragma unroll
    for (int i = 0; i < RM; ++i) fa[i] = decode_frag(second ? ra[i].y : ra[i].x, second ? sa[i].y : sa[i].x);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      const f16x8 fb = decode_frag(second ? rb[j].y : rb[j].x, second ? sbv[j].y : sbv[j].x);
#pragma unroll
      for (int i = 0; i < RM; ++i)
        acc[i][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa[i]),
                                 reinterpret_cast<const uint16_t*>(&fb), acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step s (stage s%2): stage the block fetched during step s-1 (K step
  // s+1) into stage (s+1)%2, which nobody reads since the last barrier;
  // fetch the block of step s+2; multiply slices 0 and 1; barrier; read the
  // raw fragments of stage (s+1)%2.  A fetch thus has one whole step to
  // arrive.  Two workgroups share a CU, so one workgroup's decode and LDS
  // phases overlap the other's MFMAs.  Steps past the end fetch padding and
  // stage it into a stage that is never read again.
  const int nsteps = (t.kb_end - t.kb_begin + KB - 1) / KB;
  if (nsteps > 0) {
    fetch();
    stage_block(0);
    fetch();
    __syncthreads();
    read_raw(0);
    for (int s = 0; s < nsteps; ++s) {
      const int nxt = (s + 1) & 1;
      stage_block(nxt);
      fetch();
      __builtin_amdgcn_sched_barrier(0);
      slice(false);
      slice(true);
      __syncthreads();
      read_raw(nxt);
    }
  }
  store_tile<OP, MT, NT, KB, WTM, WTN, RM, RN>(p, t, acc, lane, wm, wn);
}

// The k-blocks kb0, kb0 + KB, kb0 + 2 KB, ... of one staging thread, walked
// with additions only.  kb splits into (outer, mid, inner) as in
// TileCtx::locate; the block index and the source position are affine in the
// three, and when inner's extent is at least KB a step carries at most once
// into mid and once into outer.
template <int OP, int MT, int NT, int KB>
struct KWalk {
  uint32_t lim;            // k-blocks of this thread's range left at step 0 (kb_end - kb0)
  uint32_t inner, mid, blk;
  uint32_t d_in, d_mid;
  uint32_t s_step, s_c1, s_c2;  // block increments: per step, carry into mid, carry into outer
  int y, x, x_c1, y_c2, x_c2;   // source position and its increments on carries
  uint32_t hlim, wlim;          // position bounds (all ones: no spatial gather)

  __device__ __forceinline__ void init(const ConvParams& p, const TileCtx<OP, MT, NT, KB>& t) {
    const uint32_t kb0 = static_cast<uint32_t>(t.kb_begin + t.kbl);
    lim = (t.in_range && static_cast<int>(kb0) < t.kb_end) ? static_cast<uint32_t>(t.kb_end) - kb0 : 0u;
    const int cbin = p.c_in >> 3, cbout = p.c_out >> 3;
    int e_in, e_mid, s_in, s_mid, s_out, base;
    int sx1 = 0, sy2 = 0, sx2 = 0;
    hlim = ~0u; wlim = ~0u;
    if constexpr (OP == OP_FWD) {
      e_in = cbin; e_mid = p.k_w;
      if (t.is_a) { s_in = 1; s_mid = cbout * cbin; s_out = p.k_w * s_mid; base = t.gblk * cbin; }
      else {
        s_in = p.nb; s_mid = cbin * p.nb; s_out = p.w * s_mid;
        base = (t.sp_y * p.w + t.sp_x) * s_mid + t.col_nb;
        sx1 = 1; sy2 = 1; sx2 = -p.k_w;
        hlim = p.h; wlim = p.w;
      }
    } else if constexpr (OP == OP_DGRAD) {
      e_in = cbout; e_mid = t.nkw;
      if (t.is_a) {
        s_in = cbin; s_mid = p.sw * cbout * cbin; s_out = p.sh * p.k_w * cbout * cbin;
        base = (t.kh0 * p.k_w + t.kw0) * cbout * cbin + t.gblk;
      } else {
        s_in = p.nb; s_mid = -cbout * p.nb; s_out = -p.wo * cbout * p.nb;
        base = (t.sp_y * p.wo + t.sp_x) * cbout * p.nb + t.col_nb;
        sx1 = -1; sy2 = -1; sx2 = t.nkw;
        hlim = p.ho; wlim = p.wo;
      }
    } else {
      e_in = p.nb; e_mid = p.wo;
      if (t.is_a) { s_in = 1; s_mid = cbout * p.nb; s_out = p.wo * s_mid; base = t.gblk * p.nb; }
      else {
        s_in = 1; s_mid = p.sw * cbin * p.nb; s_out = p.sh * p.w * cbin * p.nb;
        base = (t.sp_y * p.w + t.sp_x) * cbin * p.nb + t.col_cib * p.nb;
        sx1 = p.sw; sy2 = p.sh; sx2 = -p.wo * p.sw;
        hlim = p.h; wlim = p.w;
      }
    }
    d_in = static_cast<uint32_t>(e_in);
    d_mid = static_cast<uint32_t>(e_mid > 0 ? e_mid : 1);
    const uint32_t outer_all = kb0 / d_in;
    inner = kb0 - outer_all * d_in;
    const uint32_t outer = outer_all / d_mid;
    mid = outer_all - outer * d_mid;
    blk = static_cast<uint32_t>(base) + outer * static_cast<uint32_t>(s_out) + mid * static_cast<uint32_t>(s_mid) +
          inner * static_cast<uint32_t>(s_in);
    // operands without a spatial gather stay at (0, 0)
    const bool gather = hlim != ~0u;
    y = (gather ? t.sp_y : 0) + static_cast<int>(outer) * sy2;
    x = (gather ? t.sp_x : 0) + static_cast<int>(mid) * sx1;
    s_step = static_cast<uint32_t>(KB * s_in);
    s_c1 = static_cast<uint32_t>(s_mid - e_in * s_in);
    s_c2 = static_cast<uint32_t>(s_out - e_mid * s_mid);
    x_c1 = sx1; y_c2 = sy2; x_c2 = sx2;
  }

  // the block of step s (s * KB < lim and inside the source) and advance
  __device__ __forceinline__ bool next(uint32_t s_kb, uint32_t& b) {
    const bool ok = (s_kb < lim) & (static_cast<uint32_t>(y) < hlim) & (static_cast<uint32_t>(x) < wlim);
    b = blk;
    inner += KB;
    blk += s_step;
    const bool c1 = inner >= d_in;
    inner = c1 ? inner - d_in : inner;
    mid = c1 ? mid + 1u : mid;
    blk = c1 ? blk + s_c1 : blk;
    x = c1 ? x + x_c1 : x;
    const bool c2 = mid >= d_mid;
    mid = c2 ? 0u : mid;
    blk = c2 ? blk + s_c2 : blk;
    y = c2 ? y + y_c2 : y;
    x = c2 ? x + x_c2 : x;
    return ok;
  }
};

// True when every step of KWalk carries at most once: the innermost extent
// of the K split (input channel blocks, output channel blocks, batch blocks)
// is at least the K step.
inline bool kwalk_ok(int op, const ConvParams& p, int kb) {
  const int e_in = op == OP_FWD ? p.c_in / 8 : op == OP_DGRAD ? p.c_out / 8 : p.nb;
  return e_in >= kb;
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// E2M1, 256x256 tile, 4 waves of 128x128, one workgroup per CU (the 256
// accumulator registers of a wave fill the AGPR file).  LDS holds the raw
// 4-bit codes of two K steps; each wave decodes its MFMA fragments from
// them (conversion with the block scale's exponent, then a packed multiply
// by its mantissa factor: exact in fp16).
//
// Per stage and operand, 32 pitches of 136 bytes (the 8-byte pad staggers
// the banks):
//   block rows along M/N (fwd A, wgrad A and B): 32 line blocks of 8 lines;
//     a line is 16 bytes, the 4 k-blocks of one row in the order 0, 2, 1, 3,
//     so that an 8-byte read gives k-block (lane/32) of both MFMA k-slices;
//   block rows along K (fwd B, dgrad A and B): 32 k rows of 256 codes, the
//     rows of k-block kb at pitches 8 * slot(kb); the transposing LDS read
//     (16x16 4-bit transpose within each group of 16 lanes) turns the rows
//     of 16 lanes into the k-runs of 16 columns.
// Scale words (fp32 exponent of the block scale | fp16 mantissa factor) come
// from a 256-entry table; padding blocks take entry 0, whose word is 0, so
// that their codes, whatever they are, decode to zero.
//
// Block fetches run two steps ahead in two register sets; the loop is
// unrolled twice so that sets and stages are static.
template <int OP>
__global__ __launch_bounds__(256) void k_conv4w(const ConvParams p) {
  constexpr int MT = 256, NT = 256, WM = 2, KB = 4;
  constexpr int WTM = 128, WTN = 128, RM = 4, RN = 4;
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);
  constexpr int PITCH = 136, OPND = 32 * PITCH, SCL = 32 * 16;
  constexpr int A_C = 0, B_C = OPND, A_S = 2 * OPND, B_S = 2 * OPND + SCL;
  constexpr int STAGE = 2 * OPND + 2 * SCL;
  constexpr int LUT = 2 * STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE + 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx<OP, MT, NT, KB> t;
  if (!t.init(p, tid)) return;
  const bool is_a = t.is_a;

  *reinterpret_cast<uint32_t*>(lds + LUT + tid * 4) = scale_word(static_cast<uint32_t>(tid));

  // this thread's staging addresses (every thread stages one block a step)
  const int slot = ((t.kbl & 1) << 1) | ((t.kbl >> 1) & 1);
  const bool rows = is_a ? A_ROWS : B_ROWS;  // uniform per wave
  const int st_code = (is_a ? A_C : B_C) + (rows ? t.lblk * PITCH + slot * 4 : slot * 8 * PITCH + t.lblk * 4);
  const int st_scale = (is_a ? A_S : B_S) + t.lblk * 16 + slot * 4;

  const uint8_t* my_codes = is_a ? p.a_codes : p.b_codes;
  const uint8_t* my_scales = is_a ? p.a_scales : p.b_scales;
  KWalk<OP, MT, NT, KB> walk;
  walk.init(p, t);
  uint32_t s_fetch = 0;  // k offset (s * KB) of the next fetch
  auto fetch = [&](RawBlock<FMT_E2M1>& g) {
    uint32_t blk;
    const bool ok = walk.next(s_fetch, blk);
    g.load(my_codes, my_scales, blk, ok);
    s_fetch += KB;
  };
  uint32_t sws;  // scale word of the block being staged
  auto lookup_scale = [&](const RawBlock<FMT_E2M1>& g) {
    sws = *reinterpret_cast<const uint32_t*>(lds + LUT + ((g.scale & g.mask) << 2));
  };
  auto write_rows = [&](const RawBlock<FMT_E2M1>& g, uint8_t* base, int r0) {
    if constexpr (A_ROWS == B_ROWS) {
#pragma unroll
      for (int r = r0; r < r0 + 4; ++r)
        *reinterpret_cast<uint32_t*>(base + st_code + r * (A_ROWS ? 16 : PITCH)) = g.w[r];
    } else {
      if (__builtin_amdgcn_readfirstlane(static_cast<int>(rows))) {
#pragma unroll
        for (int r = r0; r < r0 + 4; ++r) *reinterpret_cast<uint32_t*>(base + st_code + r * 16) = g.w[r];
      } else {
#pragma unroll
        for (int r = r0; r < r0 + 4; ++r) *reinterpret_cast<uint32_t*>(base + st_code + r * PITCH) = g.w[r];
      }
    }
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment read addresses (fragment i adds i * 4 pitches in the line
  // layout, i * 16 bytes in the k-row layout, i * 64 bytes of scale words)
  const int l32 = lane & 31, half = lane >> 5;
  const int line_off = (l32 >> 3) * PITCH + (l32 & 7) * 16 + half * 8;
  const int krow_off = (((lane >> 5) * 16) + (lane & 15)) * PITCH + ((lane >> 4) & 1) * 8;
  const int a_code = A_C + (A_ROWS ? wm * 16 * PITCH + line_off : krow_off + wm * 64);
  const int b_code = B_C + (B_ROWS ? wn * 16 * PITCH + line_off : krow_off + wn * 64);
  const int a_scale = A_S + (wm * 16 + (l32 >> 3)) * 16 + half * 8;
  const int b_scale = B_S + (wn * 16 + (l32 >> 3)) * 16 + half * 8;
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  u32x2 ra[RM], sa[RM], rb[RN], sbv[RN];  // raw fragments of a stage (.x slice 0, .y slice 1)
  auto read_code = [&](const uint8_t* q, bool line) -> u32x2 {
    if (line) return *reinterpret_cast<const u32x2*>(q);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2*)(q)));
  };
  auto read_raw = [&](const uint8_t* base) {
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      ra[i] = read_code(base + a_code + i * (A_ROWS ? 4 * PITCH : 16), A_ROWS);
      sa[i] = *reinterpret_cast<const u32x2*>(base + a_scale + i * 64);
    }
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      rb[j] = read_code(base + b_code + j * (B_ROWS ? 4 * PITCH : 16), B_ROWS);
      sbv[j] = *reinterpret_cast<const u32x2*>(base + b_scale + j * 64);
    }
  };
  f16x8 fa0[RM], fa1[RM];  // A fragments of slice 0 and slice 1

  // One column j of a slice: 4 MFMAs with the B fragment fb, then the work
  // item placed after them; a scheduling barrier closes the group.
  auto column = [&](const f16x8 (&fa)[RM], const f16x8& fb, int j, auto&& work) {
#pragma unroll
    for (int i = 0; i < RM; ++i)
      acc[i][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa[i]),
                               reinterpret_cast<const uint16_t*>(&fb), acc[i][j]);
    work();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Step s (fragments of stage s%2 in registers, slice-0 A decoded; set G
  // holds the block of step s+1):
  //   slice 0: decode the slice-1 A fragments and each column's B fragment;
  //            stage G into stage (s+1)%2 (free since the barrier of step
  //            s-1), then refill G with the block of step s+3
  //   slice 1: decode the B fragments, barrier, read stage (s+1)%2, decode
  //            its slice-0 A fragments
  auto step = [&](auto nxt_c, RawBlock<FMT_E2M1>& G) {
    constexpr int NXT = decltype(nxt_c)::value;
    uint8_t* nbase = lds + NXT * STAGE;
    column(fa0, decode_frag(rb[0].x, sbv[0].x), 0, [&] {
      fa1[0] = decode_frag(ra[0].y, sa[0].y);
      lookup_scale(G);
      write_rows(G, nbase, 0);
    });
    column(fa0, decode_frag(rb[1].x, sbv[1].x), 1, [&] {
      fa1[1] = decode_frag(ra[1].y, sa[1].y);
      write_rows(G, nbase, 4);
    });
    column(fa0, decode_frag(rb[2].x, sbv[2].x), 2, [&] {
      fa1[2] = decode_frag(ra[2].y, sa[2].y);
      fetch(G);
    });
    column(fa0, decode_frag(rb[3].x, sbv[3].x), 3, [&] {
      fa1[3] = decode_frag(ra[3].y, sa[3].y);
      *reinterpret_cast<uint32_t*>(nbase + st_scale) = sws;
    });
    f16x8 fb1, fb2, fb3;
    column(fa1, decode_frag(rb[0].y, sbv[0].y), 0, [&] {
      fb1 = decode_frag(rb[1].y, sbv[1].y);
      fb2 = decode_frag(rb[2].y, sbv[2].y);
    });
    column(fa1, fb1, 1, [&] {
      fb3 = decode_frag(rb[3].y, sbv[3].y);
      __syncthreads();
      read_raw(nbase);
    });
    column(fa1, fb2, 2, [&] {
      fa0[0] = decode_frag(ra[0].x, sa[0].x);
      fa0[1] = decode_frag(ra[1].x, sa[1].x);
    });
    column(fa1, fb3, 3, [&] {
      fa0[2] = decode_frag(ra[2].x, sa[2].x);
      fa0[3] = decode_frag(ra[3].x, sa[3].x);
    });
  };

  const int nsteps = (t.kb_end - t.kb_begin + KB - 1) / KB;
  if (nsteps > 0) {
    RawBlock<FMT_E2M1> g0, g1;  // blocks of even and odd steps
    fetch(g0);
    fetch(g1);
    __syncthreads();  // scale-word table
    lookup_scale(g0);
    write_rows(g0, lds, 0);
    write_rows(g0, lds, 4);
    *reinterpret_cast<uint32_t*>(lds + st_scale) = sws;
    fetch(g0);
    __syncthreads();
    read_raw(lds);
#pragma unroll
    for (int i = 0; i < RM; ++i) fa0[i] = decode_frag(ra[i].x, sa[i].x);
    // an odd step count runs one more step, on padding blocks only (zero
    // scale words: it adds exact zeros)
    for (int s = 0; s < nsteps; s += 2) {
      step(IC<1>{}, g1);
      step(IC<0>{}, g0);
    }
  }
  store_tile<OP, MT, NT, KB, WTM, WTN, RM, RN>(p, t, acc, lane, wm, wn);
}

// dW[co][ci][kh][kw] = T_dy * T_x * (sum over splits of the partials
// [split][co][(kh, kw, ci)]).  A thread owns 4 consecutive outputs (16-byte
// loads, whole 1 KiB rows per wave) and one of G split groups: group g sums
// splits g, g+G, g+2G, ... in that order; the G group sums are combined in
// LDS in group order.  The summation order depends only on the shape, so
// the result does not depend on timing.  G (1..64) is chosen so that small
// outputs still spread over enough threads.
template <int G>
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float4* __restrict__ ws, int splits, int64_t quads,
                                                      int ncol, int c_in, int k_h, int k_w,
                                                      const float* __restrict__ ta,
                                                      const float* __restrict__ tb, float* __restrict__ dw) {
  constexpr int QPW = 256 / G;  // output quads per workgroup
  const int g = threadIdx.x / QPW, qi = threadIdx.x - g * QPW;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * QPW + qi;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (q < quads) {
    int z = g;
    for (; z + 3 * G < splits; z += 4 * G) {  // 4 loads in flight, summed in split order
      const float4 a = ws[static_cast<int64_t>(z) * quads + q];
      const float4 b = ws[static_cast<int64_t>(z + G) * quads + q];
      const float4 c = ws[static_cast<int64_t>(z + 2 * G) * quads + q];
      const float4 d = ws[static_cast<int64_t>(z + 3 * G) * quads + q];
      s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
      s.x += b.x; s.y += b.y; s.z += b.z; s.w += b.w;
      s.x += c.x; s.y += c.y; s.z += c.z; s.w += c.w;
      s.x += d.x; s.y += d.y; s.z += d.z; s.w += d.w;
    }
    for (; z < splits; z += G) {
      const float4 a = ws[static_cast<int64_t>(z) * quads + q];
      s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
    }
  }
  if constexpr (G > 1) {
    __shared__ float4 part[G][QPW];
    part[g][qi] = s;
    __syncthreads();
    if (g != 0) return;
#pragma unroll 4
    for (int k = 1; k < G; ++k) {
      const float4 a = part[k][qi];
      s.x += a.x; s.y += a.y; s.z += a.z; s.w += a.w;
    }
  }
  if (q >= quads) return;
  const float scale = (*ta) * (*tb);
  // columns 4r..4r+3 of output row co: one tap, 4 consecutive input channels
  const int64_t idx = q * 4;
  const int co = static_cast<int>(idx / ncol), j = static_cast<int>(idx - static_cast<int64_t>(co) * ncol);
  const int tap = j / c_in, ci = j - tap * c_in;
  const int taps = k_h * k_w;
  float* out = dw + (static_cast<int64_t>(co) * c_in + ci) * taps + tap;
  out[0] = s.x * scale;
  out[taps] = s.y * scale;
  out[2 * taps] = s.z * scale;
  out[3 * taps] = s.w * scale;
}

// ---- tile selection and launch -------------------------------------------

struct Tile {
  int mt, nt, wm, waves, kb;
};

// Candidate tiles (MT, NT, waves along M, waves, k-blocks per stage), largest
// first.  A wave tile is a grid of 32x32 MFMAs; KB is the largest even count
// with (MT/8 + NT/8) * KB <= threads.
constexpr Tile kTiles[] = {{256, 256, 2, 4, 4}, {128, 256, 2, 4, 4}, {128, 128, 2, 4, 8},
                           {64, 256, 2, 4, 6},  {64, 128, 2, 4, 10}, {64, 64, 2, 4, 16},
                           {32, 256, 1, 4, 6},  {32, 128, 1, 4, 12}, {64, 32, 2, 2, 10},
                           {32, 64, 1, 2, 10}};

// Tile heights never exceed the GEMM's rows rounded up to a tile height.
// fwd / dgrad: the largest tile that still gives 2048 waves (two 4-wave
// workgroups per CU); else the one reaching the most CUs, preferring the
// larger tile.  The K loop of a small layer is latency-bound, so spreading
// it over more CUs beats operand reuse inside a workgroup.
int mt_cap(int64_t M) { return M > 128 ? 256 : M > 64 ? 128 : M > 32 ? 64 : 32; }

bool tile_ok(const Tile&, int) { return true; }

Tile pick_tile(int64_t M, int64_t ncols, int64_t zdim, int fmt) {
  const int cap = mt_cap(M);
  Tile best = {0, 0, 0, 0, 0};
  int64_t best_reach = -1;
  for (const Tile& t : kTiles) {
    if (t.mt > cap || !tile_ok(t, fmt)) continue;
    const int64_t wgs = ((M + t.mt - 1) / t.mt) * ((ncols + t.nt - 1) / t.nt) * zdim;
    if (wgs * t.waves >= 2048) return t;
    const int64_t reach = wgs < 256 ? wgs : 256;
    if (reach > best_reach) {
      best = t;
      best_reach = reach;
    }
  }
  return best;
}

// wgrad: split K supplies the parallelism, so the tile is chosen for operand
// reuse: the largest one whose share of useful (unpadded) outputs is within
// 3/4 of the best share any tile reaches.
Tile pick_wgrad_tile(int64_t M, int64_t ncols, int fmt) {
  const int cap = mt_cap(M);
  double best_eff = 0.0;
  for (const Tile& t : kTiles) {
    if (t.mt > cap || !tile_ok(t, fmt)) continue;
    const double eff = static_cast<double>(M * ncols) /
                       (static_cast<double>((M + t.mt - 1) / t.mt * t.mt) * ((ncols + t.nt - 1) / t.nt * t.nt));
    if (eff > best_eff) best_eff = eff;
  }
  for (const Tile& t : kTiles) {
    if (t.mt > cap || !tile_ok(t, fmt)) continue;
    const double eff = static_cast<double>(M * ncols) /
                       (static_cast<double>((M + t.mt - 1) / t.mt * t.mt) * ((ncols + t.nt - 1) / t.nt * t.nt));
    if (eff * 4.0 >= best_eff * 3.0) return t;
  }
  return kTiles[1];
}

// Reduces the per-wave slots of a producer-fused fwd into slot 0 (one
// workgroup; 0 when there are no slots).
__global__ __launch_bounds__(1024) void k_amax_finish(uint32_t* __restrict__ w, int64_t nslots) {
  uint32_t m = 0;
  for (int64_t i = threadIdx.x; i < nslots; i += 1024) m = max(m, w[1 + i]);
  for (int off = 32; off > 0; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off)));
  __shared__ uint32_t wmax[16];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 1; k < 16; ++k) m = max(m, wmax[k]);
    w[0] = m;
  }
}

template <int OP, int FMT, int MT, int NT, int WM, int WAVES, int KB>
void launch_tile(const ConvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_conv<OP, FMT, MT, NT, WM, WAVES, KB>), grid, dim3(WAVES * 64), 0, s, p);
}

template <int OP, int MT, int NT, int WM, int WAVES>
void launch_tile4(const ConvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_conv4<OP, MT, NT, WM, WAVES>), grid, dim3(WAVES * 64), 0, s, p);
}

template <int OP, int FMT>
void launch_fmt(const ConvParams& p, const Tile& t, dim3 grid, hipStream_t s) {
  // E2M1 on the 4-k-block tiles: codes in LDS, decoded at fragment read
  if constexpr (FMT == FMT_E2M1) {
    if (t.mt == 256 && kwalk_ok(OP, p, 4)) {
      hipLaunchKernelGGL((k_conv4w<OP>), grid, dim3(256), 0, s, p);
      return;
    }
    if (t.mt == 128 && t.nt == 256) return launch_tile4<OP, 128, 256, 2, 4>(p, grid, s);
  }
  if (t.mt == 256) launch_tile<OP, FMT, 256, 256, 2, 4, 4>(p, grid, s);
  else if (t.mt == 128 && t.nt == 256) launch_tile<OP, FMT, 128, 256, 2, 4, 4>(p, grid, s);
  else if (t.mt == 128) launch_tile<OP, FMT, 128, 128, 2, 4, 8>(p, grid, s);
  else if (t.mt == 64 && t.nt == 256) launch_tile<OP, FMT, 64, 256, 2, 4, 6>(p, grid, s);
  else if (t.mt == 64 && t.nt == 128) launch_tile<OP, FMT, 64, 128, 2, 4, 10>(p, grid, s);
  else if (t.mt == 64 && t.nt == 64) launch_tile<OP, FMT, 64, 64, 2, 4, 16>(p, grid, s);
  else if (t.mt == 64) launch_tile<OP, FMT, 64, 32, 2, 2, 10>(p, grid, s);
  else if (t.nt == 256) launch_tile<OP, FMT, 32, 256, 1, 4, 6>(p, grid, s);
  else if (t.nt == 128) launch_tile<OP, FMT, 32, 128, 1, 4, 12>(p, grid, s);
  else launch_tile<OP, FMT, 32, 64, 1, 2, 10>(p, grid, s);
}

template <int OP>
void launch_op(const ConvParams& p, int fmt, const Tile& t, dim3 grid, hipStream_t s) {
  switch (fmt) {
    case FMT_E2M1: launch_fmt<OP, FMT_E2M1>(p, t, grid, s); break;
    case FMT_E2M3: launch_fmt<OP, FMT_E2M3>(p, t, grid, s); break;
    default: launch_fmt<OP, FMT_E4M3>(p, t, grid, s); break;
  }
}

ConvParams base_params(const Geom& g) {
  ConvParams p{};
  p.n = g.n; p.c_in = g.c_in; p.c_out = g.c_out; p.h = g.h; p.w = g.w;
  p.k_h = g.k_h; p.k_w = g.k_w; p.sh = g.sh; p.sw = g.sw; p.ph = g.ph; p.pw = g.pw;
  p.ho = g.ho; p.wo = g.wo; p.nb = g.n / 8;
  return p;
}

// Weight gradient: tile and split count.  At least 4 K steps per split.
struct WgradPlan {
  Tile t;
  int splits;
};

WgradPlan wgrad_plan(const Geom& g) {
  const int64_t kb_total = static_cast<int64_t>(g.ho) * g.wo * (g.n / 8);
  const int64_t ncol = static_cast<int64_t>(g.k_h) * g.k_w * g.c_in;
  const Tile t = pick_wgrad_tile(g.c_out, ncol, g.fmt);
  const int64_t ksteps = (kb_total + t.kb - 1) / t.kb;
  const int64_t tiles = ((g.c_out + t.mt - 1) / t.mt) * ((ncol + t.nt - 1) / t.nt);
  // About one round of workgroups: 1024 waves, or 2048 for the 128x256 E2M1
  // tile, which runs two workgroups per CU.  More splits shorten each K loop
  // but add partials to write and reduce (a sweep over the ResNet stacks put
  // the optimum there).  Rounded down: a last, nearly empty round of
  // workgroups costs a full one.
  const int64_t target_waves = (g.fmt == FMT_E2M1 && t.mt == 128 && t.nt == 256) ? 2048 : 1024;
  int64_t splits = (target_waves / t.waves) / tiles;
  const int64_t max_by_k = ksteps / 4;
  if (splits > max_by_k) splits = max_by_k;
  if (splits < 1) splits = 1;
  if (splits > 65535) splits = 65535;
  return {t, static_cast<int>(splits)};
}

// Forward launch geometry: tile, grid and waves per workgroup.
struct FwdPlan {
  Tile t;
  dim3 grid;
};
FwdPlan fwd_plan(const Geom& g, const ConvParams& p) {
  const Tile t = pick_tile(p.M, static_cast<int64_t>(p.ncb) * 8, 1, g.fmt);
  return {t, dim3((p.ncb * 8 + t.nt - 1) / t.nt, (p.M + t.mt - 1) / t.mt, 1)};
}

ConvParams fwd_params(const Geom& g) {
  ConvParams p = base_params(g);
  p.M = g.c_out;
  p.ncb = g.ho * g.wo * (g.n / 8);
  p.kb_total = g.k_h * g.k_w * (g.c_in / 8);
  return p;
}

}  // namespace

size_t fwd_amax_bytes(const Geom& g) {
  const ConvParams p = fwd_params(g);
  if (p.ncb == 0) return 4;
  const FwdPlan pl = fwd_plan(g, p);
  return 4 * (1 + static_cast<size_t>(pl.grid.x) * pl.grid.y * pl.grid.z * pl.t.waves);
}

hipError_t launch_conv_fwd(const Geom& g, const mx_qtensor* wq, const mx_qtensor* xq, float* y,
                           float* y_amax, hipStream_t s) {
  ConvParams p = fwd_params(g);
  p.a_codes = static_cast<const uint8_t*>(wq->codes); p.a_scales = wq->scales; p.a_t = wq->tensor_scale;
  p.b_codes = static_cast<const uint8_t*>(xq->codes); p.b_scales = xq->scales; p.b_t = xq->tensor_scale;
  p.out = y;
  p.amax_out = reinterpret_cast<uint32_t*>(y_amax);
  int64_t nslots = 0;
  if (p.ncb > 0) {
    const FwdPlan pl = fwd_plan(g, p);
    nslots = static_cast<int64_t>(pl.grid.x) * pl.grid.y * pl.grid.z * pl.t.waves;
    launch_op<OP_FWD>(p, g.fmt, pl.t, pl.grid, s);
  }
  if (y_amax != nullptr)
    hipLaunchKernelGGL(k_amax_finish, dim3(1), dim3(1024), 0, s, p.amax_out, nslots);
  return hipGetLastError();
}

hipError_t launch_conv_dgrad(const Geom& g, const mx_qtensor* wq, const mx_qtensor* dyq, float* dx,
                             hipStream_t s) {
  ConvParams p = base_params(g);
  p.M = g.c_in;
  const int hp_max = (g.h + g.sh - 1) / g.sh, wp_max = (g.w + g.sw - 1) / g.sw;
  p.ncb = hp_max * wp_max * (g.n / 8);
  p.kb_total = 0;  // per phase, computed in the kernel
  p.a_codes = static_cast<const uint8_t*>(wq->codes); p.a_scales = wq->scales; p.a_t = wq->tensor_scale;
  p.b_codes = static_cast<const uint8_t*>(dyq->codes); p.b_scales = dyq->scales; p.b_t = dyq->tensor_scale;
  p.out = dx;
  if (p.ncb == 0) return hipSuccess;
  const Tile t = pick_tile(p.M, static_cast<int64_t>(p.ncb) * 8, g.sh * g.sw, g.fmt);
  dim3 grid((p.ncb * 8 + t.nt - 1) / t.nt, (p.M + t.mt - 1) / t.mt, g.sh * g.sw);
  launch_op<OP_DGRAD>(p, g.fmt, t, grid, s);
  return hipGetLastError();
}

size_t wgrad_workspace_bytes(const Geom& g) {
  const WgradPlan pl = wgrad_plan(g);
  return static_cast<size_t>(pl.splits) * g.c_out * g.k_h * g.k_w * g.c_in * sizeof(float);
}

hipError_t launch_conv_wgrad(const Geom& g, const mx_qtensor* dyq, const mx_qtensor* xq, float* dw,
                             void* workspace, hipStream_t s) {
  ConvParams p = base_params(g);
  const WgradPlan pl = wgrad_plan(g);
  p.M = g.c_out;
  p.ncol = g.k_h * g.k_w * g.c_in;
  p.ncb = p.ncol / 8;
  p.kb_total = g.ho * g.wo * (g.n / 8);
  const int ksteps = (p.kb_total + pl.t.kb - 1) / pl.t.kb;
  p.ks_split = (ksteps + pl.splits - 1) / pl.splits;
  p.a_codes = static_cast<const uint8_t*>(dyq->codes); p.a_scales = dyq->scales; p.a_t = dyq->tensor_scale;
  p.b_codes = static_cast<const uint8_t*>(xq->codes); p.b_scales = xq->scales; p.b_t = xq->tensor_scale;
  p.out = static_cast<float*>(workspace);
  dim3 grid((p.ncol + pl.t.nt - 1) / pl.t.nt, (p.M + pl.t.mt - 1) / pl.t.mt, pl.splits);
  launch_op<OP_WGRAD>(p, g.fmt, pl.t, grid, s);
  // ncol = Kh*Kw*C_in is a multiple of 8: whole quads of outputs
  const int64_t quads = static_cast<int64_t>(p.M) * p.ncol / 4;
  int gsplit = 1;  // split groups: at least 2^18 threads where the splits allow
  while (gsplit < 64 && gsplit < pl.splits && quads * gsplit < (int64_t{1} << 18)) gsplit *= 2;
  const unsigned rg = static_cast<unsigned>((quads + 256 / gsplit - 1) / (256 / gsplit));
  const float4* wsq = static_cast<const float4*>(workspace);
  auto red = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(rg), dim3(256), 0, s, wsq, pl.splits, quads, p.ncol, g.c_in, g.k_h, g.k_w,
                       dyq->tensor_scale, xq->tensor_scale, dw);
  };
  switch (gsplit) {
    case 1: red(k_wgrad_reduce<1>); break;
    case 2: red(k_wgrad_reduce<2>); break;
    case 4: red(k_wgrad_reduce<4>); break;
    case 8: red(k_wgrad_reduce<8>); break;
    case 16: red(k_wgrad_reduce<16>); break;
    case 32: red(k_wgrad_reduce<32>); break;
    default: red(k_wgrad_reduce<64>); break;
  }
  return hipGetLastError();
}

}  // namespace mx
