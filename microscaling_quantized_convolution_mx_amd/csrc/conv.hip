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
// Kernel shape: 256 threads (4 wave64), tile MT x NT, K step 32 (four 8-wide
// k-blocks), two LDS stages.  Each thread fetches at most one quantized block
// per stage, decodes it and writes its eight 8-value K-lines to LDS as
// 16-byte rows [line][k] (k contiguous), which is exactly the operand layout
// of v_mfma_f32_32x32x16_bf16 (lane l: row/col l%32, K slots 8*(l/32)..+7).
#include "internal.h"
#include "mx_formats.h"

namespace mx {
namespace {

constexpr int kThreads = 256;
constexpr int KT = 32;          // K per LDS stage
constexpr int LDS_STRIDE = 40;  // bf16 per LDS line: 32 + 8 padding (80 B) against bank conflicts

enum { OP_FWD = 0, OP_DGRAD = 1, OP_WGRAD = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

struct ConvParams {
  int32_t n, c_in, c_out, h, w, k_h, k_w, sh, sw, ph, pw, ho, wo;
  int32_t nb;         // n / 8
  int32_t M;          // GEMM rows
  int32_t ncb;        // column blocks (8 columns each) of the launch's column space
  int32_t kb_total;   // k-blocks (8 each) along K
  int32_t ks_split;   // K steps per split (wgrad)
  int32_t ncol;       // wgrad: columns of one partial (Kh*Kw*Cin)
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_t;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_t;
  float* out;
};

// Code of element (r, c) of a block from its 32-bit words (compile-time r, c
// after unrolling).
template <int FMT>
__device__ __forceinline__ uint32_t blk_code(const uint32_t* w, int r, int c) {
  constexpr int BITS = Fmt<FMT>::BITS;
  const int bit = (r * 8 + c) * BITS;
  const int wi = bit >> 5, s = bit & 31;
  uint32_t v = w[wi] >> s;
  if (s + BITS > 32) v |= w[wi + 1] << (32 - s);
  return v & ((1u << BITS) - 1u);
}

// bf16 bit pattern of the signed value code * B (exact).
template <int FMT>
__device__ __forceinline__ uint32_t dq_bf16(uint32_t code, float B) {
  using F = Fmt<FMT>;
  const float v = code_value<F>(code & ((1u << F::SIGN) - 1u)) * B;
  return (__float_as_uint(v) >> 16) | (((code >> F::SIGN) & 1u) << 15);
}

// Raw codes of one block held in registers between the global load and the
// LDS store.
template <int FMT>
struct RawBlock {
  static constexpr int WORDS = block_bytes<FMT>() / 4;
  uint32_t w[WORDS];
  uint32_t scale;
  bool valid;

  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t blk, bool ok) {
    valid = ok;
    if (ok) {
      const uint4* p = reinterpret_cast<const uint4*>(codes + blk * block_bytes<FMT>());
#pragma unroll
      for (int i = 0; i < WORDS / 4; ++i) {
        const uint4 v = p[i];
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
      }
      scale = scales[blk];
    }
  }

  // Write the block as eight K-lines of 8 bf16: line i is block row i
  // (ROWS) or block column i (!ROWS), values along the other index.
  template <bool ROWS>
  __device__ __forceinline__ void store(uint16_t* line0) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 o = make_uint4(0u, 0u, 0u, 0u);
      if (valid) {
        const float B = code_value<ScaleFmt>(scale);
        uint32_t q[4];
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const uint32_t c0 = ROWS ? blk_code<FMT>(w, i, k) : blk_code<FMT>(w, k, i);
          const uint32_t c1 = ROWS ? blk_code<FMT>(w, i, k + 1) : blk_code<FMT>(w, k + 1, i);
          q[k / 2] = dq_bf16<FMT>(c0, B) | (dq_bf16<FMT>(c1, B) << 16);
        }
        o = make_uint4(q[0], q[1], q[2], q[3]);
      }
      *reinterpret_cast<uint4*>(line0 + i * LDS_STRIDE) = o;
    }
  }
};

// Which operand block a thread stages for one K step, and where it goes.
struct Slot {
  bool is_a;      // A (rows) or B (columns) tile
  int line;       // first LDS line (A: local row, B: MT + local column)
  int kbl;        // k-block within the step (0..3)
  int gblk;       // global row-block (A) or column-block (B)
};

template <int OP, int FMT, int MT, int NT, int WM>
__global__ __launch_bounds__(kThreads) void k_conv(const ConvParams p) {
  constexpr int WN = 4 / WM;
  constexpr int WTM = MT / WM, WTN = NT / WN;
  constexpr int RM = WTM / 32, RN = WTN / 32;
  constexpr int ABLK = (MT / 8) * 4, BBLK = (NT / 8) * 4;
  static_assert(ABLK + BBLK <= kThreads, "one block per thread per stage");
  static_assert(RM >= 1 && RN >= 1, "wave tile at least 32x32");

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(MT + NT) * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int rb0 = blockIdx.y * (MT / 8);
  const int cb0 = blockIdx.x * (NT / 8);

  // ---- per-launch-z context: data-gradient phase or weight-gradient split
  int phh = 0, phw = 0, kh0 = 0, kw0 = 0, nkh = p.k_h, nkw = p.k_w, hp = 0, wp = 0;
  int kb_begin = 0, kb_end = p.kb_total;
  if constexpr (OP == OP_DGRAD) {
    // output pixels (h, w) with h = phh + sh*h', w = phw + sw*w' receive the
    // taps kh = (phh + ph) mod sh (+ sh, ...), kw likewise
    phh = blockIdx.z / p.sw;
    phw = blockIdx.z % p.sw;
    kh0 = (phh + p.ph) % p.sh;
    kw0 = (phw + p.pw) % p.sw;
    nkh = kh0 < p.k_h ? (p.k_h - kh0 + p.sh - 1) / p.sh : 0;
    nkw = kw0 < p.k_w ? (p.k_w - kw0 + p.sw - 1) / p.sw : 0;
    hp = (p.h - phh + p.sh - 1) / p.sh;
    wp = (p.w - phw + p.sw - 1) / p.sw;
    const int ncb_phase = hp * wp * p.nb;
    if (cb0 >= ncb_phase) return;
    kb_end = nkh * nkw * (p.c_out >> 3);
  } else if constexpr (OP == OP_WGRAD) {
    kb_begin = blockIdx.z * p.ks_split * 4;
    kb_end = min(p.kb_total, kb_begin + p.ks_split * 4);
    if (kb_begin > kb_end) kb_begin = kb_end;
  }
  const int ncb_launch = (OP == OP_DGRAD) ? hp * wp * p.nb : p.ncb;

  // ---- the block this thread stages every step
  Slot slot;
  slot.is_a = tid < ABLK;
  if (slot.is_a) {
    slot.line = (tid >> 2) * 8;
    slot.kbl = tid & 3;
    slot.gblk = rb0 + (tid >> 2);
  } else {
    const int t = tid - ABLK;
    slot.line = MT + (t >> 2) * 8;
    slot.kbl = t & 3;
    slot.gblk = cb0 + (t >> 2);
  }
  const bool active = tid < ABLK + BBLK;
  const bool in_range = slot.is_a ? (slot.gblk < (p.M >> 3)) : (slot.gblk < ncb_launch);

  // Column-block geometry fixed over the K loop.
  int col_ho = 0, col_wo = 0, col_nb = 0;  // FWD: output position; DGRAD: input pixel
  int col_tap_h = 0, col_tap_w = 0, col_cib = 0;  // WGRAD: tap and channel block
  if (!slot.is_a && in_range) {
    if constexpr (OP == OP_FWD) {
      const int pos = slot.gblk / p.nb;
      col_nb = slot.gblk - pos * p.nb;
      col_ho = pos / p.wo;
      col_wo = pos - col_ho * p.wo;
    } else if constexpr (OP == OP_DGRAD) {
      const int pos = slot.gblk / p.nb;
      col_nb = slot.gblk - pos * p.nb;
      const int hq = pos / wp;
      col_ho = phh + p.sh * hq;             // input row h
      col_wo = phw + p.sw * (pos - hq * wp); // input col w
    } else {
      const int cbin = p.c_in >> 3;
      const int tap = slot.gblk / cbin;
      col_cib = slot.gblk - tap * cbin;
      col_tap_h = tap / p.k_w;
      col_tap_w = tap - col_tap_h * p.k_w;
    }
  }

  // Locate the quantized block of this thread's slot for k-block kb; returns
  // false when it lies in the zero padding (or outside the GEMM).
  auto locate = [&](int kb, int64_t& blk) -> bool {
    if (!active || !in_range || kb >= kb_end) return false;
    const int cbin = p.c_in >> 3, cbout = p.c_out >> 3;
    if constexpr (OP == OP_FWD) {
      const int tap = kb / cbin, cib = kb - tap * cbin;
      if (slot.is_a) {
        blk = (static_cast<int64_t>(tap) * cbout + slot.gblk) * cbin + cib;
        return true;
      }
      const int kh = tap / p.k_w, kw = tap - kh * p.k_w;
      const int hh = col_ho * p.sh + kh - p.ph, ww = col_wo * p.sw + kw - p.pw;
      if (hh < 0 || hh >= p.h || ww < 0 || ww >= p.w) return false;
      blk = ((static_cast<int64_t>(hh) * p.w + ww) * cbin + cib) * p.nb + col_nb;
      return true;
    } else if constexpr (OP == OP_DGRAD) {
      const int ti = kb / cbout, cob = kb - ti * cbout;
      const int it = ti / nkw;
      const int kh = kh0 + p.sh * it, kw = kw0 + p.sw * (ti - it * nkw);
      if (slot.is_a) {
        blk = ((static_cast<int64_t>(kh) * p.k_w + kw) * cbout + cob) * cbin + slot.gblk;
        return true;
      }
      const int th = col_ho + p.ph - kh, tw = col_wo + p.pw - kw;  // divisible by the strides
      if (th < 0 || tw < 0) return false;
      const int ho = th / p.sh, wo = tw / p.sw;
      if (ho >= p.ho || wo >= p.wo) return false;
      blk = ((static_cast<int64_t>(ho) * p.wo + wo) * cbout + cob) * p.nb + col_nb;
      return true;
    } else {
      const int pos = kb / p.nb, nbk = kb - pos * p.nb;
      if (slot.is_a) {
        blk = (static_cast<int64_t>(pos) * cbout + slot.gblk) * p.nb + nbk;
        return true;
      }
      const int ho = pos / p.wo, wo = pos - ho * p.wo;
      const int hh = ho * p.sh + col_tap_h - p.ph, ww = wo * p.sw + col_tap_w - p.pw;
      if (hh < 0 || hh >= p.h || ww < 0 || ww >= p.w) return false;
      blk = ((static_cast<int64_t>(hh) * p.w + ww) * cbin + col_cib) * p.nb + nbk;
      return true;
    }
  };

  // A lines are block rows for FWD (co rows, ci along K) and WGRAD (co rows,
  // n along K), block columns for DGRAD (ci lines, co along K).  B lines are
  // block columns for FWD (n lines, ci along K) and DGRAD (n lines, co along
  // K), block rows for WGRAD (ci lines, n along K).
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);

  RawBlock<FMT> raw;
  auto fetch = [&](int step) {
    const int kb = kb_begin + step * 4 + slot.kbl;
    int64_t blk = 0;
    const bool ok = locate(kb, blk);
    if (slot.is_a) raw.load(p.a_codes, p.a_scales, blk, ok);
    else raw.load(p.b_codes, p.b_scales, blk, ok);
  };
  auto stage = [&](int buf) {
    if (!active) return;
    uint16_t* line0 = &lds[buf][slot.line * LDS_STRIDE + slot.kbl * 8];
    if (slot.is_a) raw.template store<A_ROWS>(line0);
    else raw.template store<B_ROWS>(line0);
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nsteps = (kb_end - kb_begin + 3) / 4;
  if (nsteps > 0) {
    fetch(0);
    stage(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const int buf = s & 1;
      if (s + 1 < nsteps) fetch(s + 1);
      const uint16_t* As = lds[buf];
      const uint16_t* Bs = lds[buf] + MT * LDS_STRIDE;
#pragma unroll
      for (int kk = 0; kk < KT / 16; ++kk) {
        const int koff = kk * 16 + (lane >> 5) * 8;
        bf16x8 af[RM], bfr[RN];
#pragma unroll
        for (int i = 0; i < RM; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * WTM + i * 32 + (lane & 31)) * LDS_STRIDE + koff);
#pragma unroll
        for (int j = 0; j < RN; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * WTN + j * 32 + (lane & 31)) * LDS_STRIDE + koff);
#pragma unroll
        for (int i = 0; i < RM; ++i)
#pragma unroll
          for (int j = 0; j < RN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (s + 1 < nsteps) stage(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: D lane layout of the 32x32 MFMA: column lane%32, rows
  // 8*(v/4) + 4*(lane/32) + v%4 for accumulator element v
  float scale = 1.0f;
  if constexpr (OP != OP_WGRAD) scale = (*p.a_t) * (*p.b_t);
  int64_t row_stride;
  if constexpr (OP == OP_WGRAD) row_stride = p.ncol;
  else row_stride = p.n;

#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int col = cb0 * 8 + wn * WTN + j * 32 + (lane & 31);  // column in the launch space
    const int cbk = col >> 3, c = col & 7;
    if (cbk >= ncb_launch) continue;
    int64_t colbase;
    if constexpr (OP == OP_FWD) {
      const int pos = cbk / p.nb, nbk = cbk - pos * p.nb;
      colbase = static_cast<int64_t>(pos) * p.c_out * p.n + nbk * 8 + c;
    } else if constexpr (OP == OP_DGRAD) {
      const int pos = cbk / p.nb, nbk = cbk - pos * p.nb;
      const int hq = pos / wp;
      const int hh = phh + p.sh * hq, ww = phw + p.sw * (pos - hq * wp);
      colbase = (static_cast<int64_t>(hh) * p.w + ww) * p.c_in * p.n + nbk * 8 + c;
    } else {
      colbase = static_cast<int64_t>(blockIdx.z) * p.M * p.ncol + col;
    }
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rb0 * 8 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < p.M) p.out[colbase + row * row_stride] = acc[i][j][v] * scale;
      }
  }
}

// dW[co][ci][kh][kw] = T_dy * T_x * sum over splits (fixed order) of the
// partial [split][co][(kh, kw, ci)].
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ ws, int splits, int M,
                                                      int ncol, int c_in, int k_h, int k_w,
                                                      const float* __restrict__ ta,
                                                      const float* __restrict__ tb, float* __restrict__ dw) {
  const int64_t total = static_cast<int64_t>(M) * ncol;
  const float scale = (*ta) * (*tb);
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int co = static_cast<int>(idx / ncol), j = static_cast<int>(idx - static_cast<int64_t>(co) * ncol);
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += ws[static_cast<int64_t>(z) * total + idx];
    const int tap = j / c_in, ci = j - tap * c_in;
    const int kh = tap / k_w, kw = tap - kh * k_w;
    dw[((static_cast<int64_t>(co) * c_in + ci) * k_h + kh) * k_w + kw] = s * scale;
  }
}

// ---- tile selection and launch -------------------------------------------

struct Tile {
  int mt, nt, wm;
};

Tile pick_tile(int M) {
  if (M >= 256) return {256, 256, 2};
  if (M >= 128) return {128, 256, 2};
  if (M >= 64) return {64, 256, 2};
  return {32, 256, 1};
}

template <int OP, int FMT, int MT, int NT, int WM>
void launch_tile(const ConvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_conv<OP, FMT, MT, NT, WM>), grid, dim3(kThreads), 0, s, p);
}

template <int OP, int FMT>
void launch_fmt(const ConvParams& p, const Tile& t, dim3 grid, hipStream_t s) {
  if (t.mt == 256) launch_tile<OP, FMT, 256, 256, 2>(p, grid, s);
  else if (t.mt == 128) launch_tile<OP, FMT, 128, 256, 2>(p, grid, s);
  else if (t.mt == 64) launch_tile<OP, FMT, 64, 256, 2>(p, grid, s);
  else launch_tile<OP, FMT, 32, 256, 1>(p, grid, s);
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

// Split count of the weight gradient: enough workgroups to cover the 256 CUs
// twice, at least 8 K steps per split.
int wgrad_splits(const Geom& g, const Tile& t) {
  const int64_t kb_total = static_cast<int64_t>(g.ho) * g.wo * (g.n / 8);
  const int64_t ksteps = (kb_total + 3) / 4;
  const int64_t ncol = static_cast<int64_t>(g.k_h) * g.k_w * g.c_in;
  const int64_t tiles = ((g.c_out + t.mt - 1) / t.mt) * ((ncol + t.nt - 1) / t.nt);
  int64_t splits = (512 + tiles - 1) / tiles;
  const int64_t max_by_k = ksteps / 8;
  if (splits > max_by_k) splits = max_by_k;
  if (splits < 1) splits = 1;
  if (splits > 65535) splits = 65535;
  return static_cast<int>(splits);
}

}  // namespace

hipError_t launch_conv_fwd(const Geom& g, const mx_qtensor* wq, const mx_qtensor* xq, float* y,
                           hipStream_t s) {
  ConvParams p = base_params(g);
  p.M = g.c_out;
  p.ncb = g.ho * g.wo * (g.n / 8);
  p.kb_total = g.k_h * g.k_w * (g.c_in / 8);
  p.a_codes = static_cast<const uint8_t*>(wq->codes); p.a_scales = wq->scales; p.a_t = wq->tensor_scale;
  p.b_codes = static_cast<const uint8_t*>(xq->codes); p.b_scales = xq->scales; p.b_t = xq->tensor_scale;
  p.out = y;
  if (p.ncb == 0) return hipSuccess;
  const Tile t = pick_tile(p.M);
  dim3 grid((p.ncb * 8 + t.nt - 1) / t.nt, (p.M + t.mt - 1) / t.mt, 1);
  launch_op<OP_FWD>(p, g.fmt, t, grid, s);
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
  const Tile t = pick_tile(p.M);
  dim3 grid((p.ncb * 8 + t.nt - 1) / t.nt, (p.M + t.mt - 1) / t.mt, g.sh * g.sw);
  launch_op<OP_DGRAD>(p, g.fmt, t, grid, s);
  return hipGetLastError();
}

size_t wgrad_workspace_bytes(const Geom& g) {
  const Tile t = pick_tile(g.c_out);
  const int splits = wgrad_splits(g, t);
  return static_cast<size_t>(splits) * g.c_out * g.k_h * g.k_w * g.c_in * sizeof(float);
}

hipError_t launch_conv_wgrad(const Geom& g, const mx_qtensor* dyq, const mx_qtensor* xq, float* dw,
                             void* workspace, hipStream_t s) {
  ConvParams p = base_params(g);
  const Tile t = pick_tile(g.c_out);
  const int splits = wgrad_splits(g, t);
  p.M = g.c_out;
  p.ncol = g.k_h * g.k_w * g.c_in;
  p.ncb = p.ncol / 8;
  p.kb_total = g.ho * g.wo * (g.n / 8);
  const int ksteps = (p.kb_total + 3) / 4;
  p.ks_split = (ksteps + splits - 1) / splits;
  p.a_codes = static_cast<const uint8_t*>(dyq->codes); p.a_scales = dyq->scales; p.a_t = dyq->tensor_scale;
  p.b_codes = static_cast<const uint8_t*>(xq->codes); p.b_scales = xq->scales; p.b_t = xq->tensor_scale;
  p.out = static_cast<float*>(workspace);
  dim3 grid((p.ncol + t.nt - 1) / t.nt, (p.M + t.mt - 1) / t.mt, splits);
  launch_op<OP_WGRAD>(p, g.fmt, t, grid, s);
  const int64_t total = static_cast<int64_t>(p.M) * p.ncol;
  int64_t rg = (total + 255) / 256;
  if (rg > 65535) rg = 65535;
  if (rg < 1) rg = 1;
  hipLaunchKernelGGL(k_wgrad_reduce, dim3(static_cast<unsigned>(rg)), dim3(256), 0, s,
                     static_cast<const float*>(workspace), splits, p.M, p.ncol, g.c_in, g.k_h, g.k_w,
                     dyq->tensor_scale, xq->tensor_scale, dw);
  return hipGetLastError();
}

}  // namespace mx
