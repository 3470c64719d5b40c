// Generic implicit-im2col convolution GEMM on microscaled operands (gfx950
// MFMA), shared by the translation units that instantiate it.
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
// has at most 8 significant bits and an exponent within bf16 range for every
// element format, so it is exactly a bf16 (and exactly an fp16 for E2M1, E2M3
// and E3M2); a product of two such values is exact in fp32.  The MFMA therefore sums exact products of the Eq. 7
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
#pragma once

#include <type_traits>
#include <utility>

#include "internal.h"
#include "mx_formats.h"

namespace mx {
namespace gemm {

enum { OP_FWD = 0, OP_DGRAD = 1, OP_WGRAD = 2 };

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
  int32_t stream_out;  // fwd / dgrad: write the output with nontemporal stores (outputs above kStreamOutBytes)
  // fwd / dgrad: column tiles per row of output positions and the band
  // height of the band order (TileCtx::init); 0: launch order
  int32_t band_tpr, band_rows;
};

// Tile of one launch: MT x NT outputs, waves along M, waves, k-blocks per stage.
struct Tile {
  int mt, nt, wm, waves, kb;
};

// Launches the generic kernel for operand formats other than the three
// uniform hot-path ones (defined in conv_mixed.hip): uniform E3M2, and
// E2M1 weights / gradients with E2M3 or E3M2 activations in the forward
// and weight-gradient GEMMs.  Returns false for a pair it does not take.
bool launch_mixed(int op, const ConvParams& p, int fmt_a, int fmt_b, const Tile& t, dim3 grid, hipStream_t s);

// Launches the 256x256 E4M3 GEMM that keeps the codes as bytes in LDS and
// decodes them at fragment read (defined in conv8.hip).  Returns false
// (nothing launched) where its K walk does not apply.
bool launch_conv8(int op, const ConvParams& p, dim3 grid, hipStream_t s);

// Launches the 256x256 GEMM of FP6 activations (E2M3 or E3M2 throughout, or
// E2M1 A with FP6 B in the forward and weight-gradient GEMMs) that fetches
// every block two K steps ahead and decodes it once into fp16 in LDS
// (defined in conv_staged.hip).  Returns false (nothing launched) for another
// format pair or where its K walk does not apply.
bool launch_staged(int op, int fmt_a, int fmt_b, const ConvParams& p, dim3 grid, hipStream_t s);

// Launches the E8M0 32x32-block GEMM on the scaled FP4 MFMA (defined in
// conv_mx.hip): tile x tile outputs per workgroup (tile 256 or 128), the
// grid as for the generic kernel; for the weight gradient p.ks_split counts
// its K steps (kMxStepBlocks 32-blocks each) per split.
void launch_mx(int op, int tile, const ConvParams& p, dim3 grid, hipStream_t s);
// 32-blocks along K per step of that kernel (each row / column block of a
// tile stages this many blocks per step)
constexpr int kMxStepBlocks = 4;

}  // namespace gemm

// The kernels have internal linkage: every translation unit that includes
// this header registers its own instantiations.
namespace {
using namespace gemm;


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


typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned int u32x6 __attribute__((ext_vector_type(6)));


// MFMA operand type: E2M1, E2M3 and E3M2 blocks decode exactly to fp16 (g*B
// lies in [2^-13, 12544] with at most 8 significant bits); E4M3 x E4M3 spans
// 2^-18 .. 2*10^5, beyond fp16's normal range, and decodes exactly to bf16.
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
// intervening K steps compute.  WORDS is the room (the larger block of
// two operand formats); load<NW> reads one block of NW words.
template <int WORDS>
struct RawWords {
  uint32_t w[WORDS];
  uint32_t scale;
  uint32_t mask;  // ~0 for a block of the tensor, 0 for padding

  template <int NW = WORDS>
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, uint32_t blk, bool ok) {
    static_assert(NW <= WORDS && NW % 4 == 0, "whole 16-byte loads within the room");
    const uint64_t b = ok ? blk : 0u;
    const uint4* p = reinterpret_cast<const uint4*>(codes + b * (4 * NW));
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
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
template <int FMT> using RawBlock = RawWords<block_bytes<FMT>() / 4>;

// Staging of one block into LDS, cut into units so that the units can be
// placed between the MFMAs of a K step.  ROWS: unit u (0..7) writes line u =
// block row u.  !ROWS: unit u (0..3) writes lines 2u and 2u+1 = block columns
// 2u, 2u+1 (a 2x2 transpose of the row pairs).  Each unit decodes what it
// writes (the FP6 formats decode 32 elements at a time: in the first unit of
// a 4-row group for ROWS, all 64 in unit 0 for !ROWS).  The raw block has
// room for WORDS words (at least the format's own).
template <int FMT, bool ROWS, int LS, int WORDS = block_bytes<FMT>() / 4>
struct Stager {
  using Raw = RawWords<WORDS>;
  static constexpr bool FP6 = Fmt<FMT>::BITS == 6;
  static constexpr int UNITS = ROWS ? 8 : 4;
  BlockScale bs;
  uint32_t mask;
  uint32_t P[8][4];  // pairs (element (r,2j), element (r,2j+1)) as two 16-bit floats
  uint16_t* p_lo;    // lines 0-3 of the block (swizzled halves, see lds_line)
  uint16_t* p_hi;    // lines 4-7

  __device__ __forceinline__ Stager(const Raw& raw, uint16_t* lo, uint16_t* hi)
      : bs(raw.scale & raw.mask), mask(raw.mask), p_lo(lo), p_hi(hi) {}

  __device__ __forceinline__ uint16_t* line_ptr(int i) const {
    return (i < 4) ? p_lo + i * LS : p_hi + (i - 4) * LS;
  }

  // pair j of row r
  template <int R, int J>
  __device__ __forceinline__ uint32_t pair(const Raw& raw) const {
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

  // FP6: rows 4G .. 4G+3 (192 consecutive bits) into P
  template <int G>
  __device__ __forceinline__ void fp6_group(const Raw& raw) {
    const _Float16 m = static_cast<_Float16>(bs.mb);
    const f16x2 m2 = {m, m};
    u32x6 src;
    src[0] = raw.w[6 * G + 0] & mask; src[1] = raw.w[6 * G + 1] & mask; src[2] = raw.w[6 * G + 2] & mask;
    src[3] = raw.w[6 * G + 3] & mask; src[4] = raw.w[6 * G + 4] & mask; src[5] = raw.w[6 * G + 5] & mask;
    const auto v = [&] {
      if constexpr (FMT == FMT_E3M2) return __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(src, bs.b);
      else return __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(src, bs.b);
    }();
    struct Words { uint32_t u[16]; };
    const Words wv = __builtin_bit_cast(Words, v);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      P[4 * G + i / 4][i % 4] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, wv.u[i]) * m2);
  }

  template <int U>
  __device__ __forceinline__ void unit(const Raw& raw) {
    if constexpr (ROWS) {
      if constexpr (FP6) {
        if constexpr (U % 4 == 0) fp6_group<U / 4>(raw);
      } else {
        P[U][0] = pair<U, 0>(raw);
        P[U][1] = pair<U, 1>(raw);
        P[U][2] = pair<U, 2>(raw);
        P[U][3] = pair<U, 3>(raw);
      }
      *reinterpret_cast<uint4*>(line_ptr(U)) = make_uint4(P[U][0], P[U][1], P[U][2], P[U][3]);
    } else {
      if constexpr (FP6) {
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
    // Band order (fwd / dgrad, where a row of output positions is a whole
    // number of column tiles): consecutive tiles walk down band_rows rows of
    // positions before moving right, so that the tiles one XCD runs at once
    // form a patch of positions whose input blocks, reused across the taps,
    // stay in that XCD's L2 (in row order the rows above and below have left
    // it by the time they are reused).  A bijection on the column tiles.
    if constexpr (OP != OP_WGRAD) {
      if (p.band_tpr > 0) {
        const int tpr = p.band_tpr, R = p.band_rows, rows = gridDim.x / tpr;
        const int b = bx / (R * tpr), off = bx - b * (R * tpr);
        const int rb = min(R, rows - b * R);
        const int c = off / rb, rr = off - c * rb;
        bx = (b * R + rr) * tpr + c;
      }
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

// Epilogue: D lane layout of the 32x32 MFMA: column lane%32, rows
// 8*(v/4) + 4*(lane/32) + v%4 for accumulator element v.  fwd / dgrad write
// the scaled outputs in place; wgrad writes unscaled split partials.
// `unit` is the value of one accumulator unit (a power of two: kernels that
// decode their operands scaled by 2^-k pass 2^2k), applied after T_a * T_b.
template <int OP, int MT, int NT, int KB, int WTM, int WTN, int RM, int RN>
__device__ __forceinline__ void store_tile(const ConvParams& p, const TileCtx<OP, MT, NT, KB>& t,
                                           const f32x16 (&acc)[RM][RN], int lane, int wm, int wn,
                                           float unit = 1.0f) {
  float scale = unit;
  if constexpr (OP != OP_WGRAD) scale = ((*p.a_t) * (*p.b_t)) * unit;
  int64_t row_stride;
  if constexpr (OP == OP_WGRAD) row_stride = p.ncol;
  else row_stride = p.n;

  uint32_t ymax = 0;  // fwd: max over the written outputs of their sign-cleared bits
  // the weight gradient's split partials are read back at once by the
  // reduce, so they always stay cacheable
  const bool stream = OP != OP_WGRAD && p.stream_out;
  auto put = [&](float* q, float v) {
    if (stream) __builtin_nontemporal_store(v, q);
    else *q = v;
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

// FMT: element format of the A operand; FMTB: that of B (the activation in
// the forward and weight-gradient GEMMs, which MicroQonv+ keeps in FP6 while
// A is FP4).  Both must decode to the same MFMA operand type.
template <int OP, int FMT, int MT, int NT, int WM, int WAVES, int KB, int FMTB = FMT>
__global__ __launch_bounds__(WAVES * 64) void k_conv(const ConvParams p) {
  constexpr int WN = WAVES / WM;
  constexpr int WTM = MT / WM, WTN = NT / WN;
  constexpr int RM = WTM / 32, RN = WTN / 32;
  constexpr int ABLK = (MT / 8) * KB, BBLK = (NT / 8) * KB;
  constexpr int NK = KB / 2;  // 16-wide MFMA K slices per stage
  constexpr int LS = Lds<KB>::LS;
  static_assert(KB % 2 == 0, "a stage is a whole number of 16-wide K slices");
  constexpr bool F16 = OperandType<FMT>::F16;
  static_assert(F16 == OperandType<FMTB>::F16, "one MFMA operand type for A and B");
  constexpr int WA = block_bytes<FMT>() / 4, WB = block_bytes<FMTB>() / 4;
  constexpr int RW = WA > WB ? WA : WB;
  using Raw = RawWords<RW>;
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
  Raw raw0, raw1;
  const uint8_t* my_codes = is_a ? p.a_codes : p.b_codes;
  const uint8_t* my_scales = is_a ? p.a_scales : p.b_scales;
  auto fetch = [&](Raw& raw) {
    uint32_t blk = 0;
    const bool ok = t.locate(p, blk);
    if constexpr (WA == WB) raw.load(my_codes, my_scales, blk, ok);
    else if (is_a) raw.template load<WA>(my_codes, my_scales, blk, ok);
    else raw.template load<WB>(my_codes, my_scales, blk, ok);
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
  using StA = Stager<FMT, A_ROWS, LS, RW>;
  using StB = Stager<FMTB, B_ROWS, LS, RW>;
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
  auto units_after = [&](auto& st, const Raw& nxt, int m, bool on) {
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
  auto run_step = [&]<int PAR>(int cur, int nstage, int dst, const Raw& nxt, Raw& fut) {
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
  auto stage_all = [&](const Raw& raw, int stage) {
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

template <int OP, int FMT, int MT, int NT, int WM, int WAVES, int KB, int FMTB>
void launch_tile(const ConvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_conv<OP, FMT, MT, NT, WM, WAVES, KB, FMTB>), grid, dim3(WAVES * 64), 0, s, p);
}

// The generic kernel at the chosen tile (one of the candidate tiles of the
// tile selection).
template <int OP, int FMT, int FMTB>
void launch_generic(const ConvParams& p, const Tile& t, dim3 grid, hipStream_t s) {
  if (t.mt == 256) launch_tile<OP, FMT, 256, 256, 2, 4, 4, FMTB>(p, grid, s);
  else if (t.mt == 128 && t.nt == 256) launch_tile<OP, FMT, 128, 256, 2, 4, 4, FMTB>(p, grid, s);
  else if (t.mt == 128) launch_tile<OP, FMT, 128, 128, 2, 4, 8, FMTB>(p, grid, s);
  else if (t.mt == 64 && t.nt == 256) launch_tile<OP, FMT, 64, 256, 2, 4, 6, FMTB>(p, grid, s);
  else if (t.mt == 64 && t.nt == 128) launch_tile<OP, FMT, 64, 128, 2, 4, 10, FMTB>(p, grid, s);
  else if (t.mt == 64 && t.nt == 64) launch_tile<OP, FMT, 64, 64, 2, 4, 16, FMTB>(p, grid, s);
  else if (t.mt == 64) launch_tile<OP, FMT, 64, 32, 2, 2, 10, FMTB>(p, grid, s);
  else if (t.nt == 256) launch_tile<OP, FMT, 32, 256, 1, 4, 6, FMTB>(p, grid, s);
  else if (t.nt == 128) launch_tile<OP, FMT, 32, 128, 1, 4, 12, FMTB>(p, grid, s);
  else launch_tile<OP, FMT, 32, 64, 1, 2, 10, FMTB>(p, grid, s);
}

}  // namespace
}  // namespace mx
