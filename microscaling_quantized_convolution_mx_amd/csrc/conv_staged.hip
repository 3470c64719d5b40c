// Convolution GEMMs with FP6 activations on the 256x256 tile, every block
// decoded once, at staging, into exact fp16 values in LDS (MicroQonv, arXiv
// 2609.28358, §IV-B): an FP6 element format (E2M3, E3M2) throughout (the FP6
// elements of §IV-E), or MicroQonv+'s pair of §IV-D / Table VI, E2M1 weights
// and gradients with FP6 activations (the forward and weight-gradient GEMMs).
//
// The thread that stages a block decodes it into g * B (FP6: two 32-value
// conversions, which apply the exponent of B; E2M1: 32 two-value
// conversions; then packed multiplies by the mantissa factor mB, see
// BlockScale), and the MFMA fragments are read from LDS as they are.  Both
// steps are exact (g * B has at most 8 significant bits and lies in
// [2^-13, 12544]), so the fp16 MFMA sums the exact products of Eq. 7.
//
// What differs from the generic kernel (conv_kernels.h), which decodes the
// same way: the A- and B-staging waves run one instruction stream (staging
// addresses and strides are data, not branches), and each block is fetched
// two K steps before its decode into one of two register sets, refilled
// right after the decode has read it.  In the generic kernel a block has
// one K step to arrive, and the 48-byte FP6 blocks, many of them from L2,
// were not covered by it: without its global loads that kernel ran ~23%
// faster.  With one instruction stream the compiler also keeps the wait for
// a fetch at the decode that needs it, instead of at the top of the step.
//
// LDS per stage and operand (fp16):
//   lines (block rows along M/N: fwd A, wgrad A and B): 256 lines of the
//     stage's 32 K values, pitch 80 bytes, line L stored at L ^ ((L >> 2) & 4)
//     (the two halves of every second 8-line block swapped): the 16-byte
//     fragment reads of 16 consecutive lines and the 16-byte staging writes
//     of 4 line blocks x 4 k-blocks each hit 16 distinct bank quads;
//   k rows (block rows along K: fwd B, dgrad A and B): 32 k rows of 256
//     fp16 columns, pitch 576 bytes, plus 64 bytes after every 8 rows.  The
//     16-bit transposing LDS read (ds_read_b64_tr_b16: within each group of
//     16 lanes, lanes 4e .. 4e+3 supply row e of a 4 x 16 matrix of 16-bit
//     values, 4 each, and lane o receives column o) gives each lane 4
//     consecutive K values of its column; two of them make an MFMA fragment.
//     A pass of 32 lanes reads 4 rows x 64 bytes at row offsets 64 bytes
//     apart modulo the 256-byte bank row, and the staging writes of 4 column
//     blocks x 4 k-blocks fall 16 and 64 bytes apart: both conflict-free.
// Tile: 4 waves of 128x128 (a wave's 16 accumulator tiles fill its 256
// AGPRs), K steps of 4 k-blocks (two 16-wide MFMA slices), four LDS
// stages (160 KB for the weight gradient, whose operands are both staged as
// lines); every fragment of a stage is read in the step before its use, so
// one barrier serves two K steps.
#include "conv_kernels.h"

namespace mx {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// The scale code of a block comes from the aligned 32-bit word of the scales
// array that holds it (the array is padded past its last block), so that the
// value carried across the K loop is a whole loaded word: a loop-carried
// byte gets a zero-extension at the top of the loop body, which waits for
// its load there.  As in RawWords, a block outside the tensor loads block 0
// and carries mask 0.
struct RawScale {
  uint32_t sword;  // scales word holding the block's scale code
  uint32_t sbit;   // bit offset of the code in sword
  uint32_t mask;   // ~0 for a block of the tensor, 0 for padding
  __device__ __forceinline__ void load(const uint8_t* scales, uint64_t b, bool ok) {
    sword = *reinterpret_cast<const uint32_t*>(scales + (b & ~static_cast<uint64_t>(3)));
    sbit = static_cast<uint32_t>(b & 3u) * 8u;
    mask = ok ? ~0u : 0u;
  }
  __device__ __forceinline__ uint32_t code() const { return __builtin_amdgcn_ubfe(sword, sbit, 8) & mask; }
};

// Raw block between its global load and its decode: two 6-word groups.  An
// FP6 block (48 bytes) fills both, each loaded by one vector load straight
// into the register tuple that the 32-value conversion reads; the address of
// group 1 passes through an empty asm statement, so that the compiler cannot
// merge the loads into 16-byte pieces that straddle the groups (the register
// copies that would then build the tuples wait for the newest loads).  An
// E2M1 block (32 bytes) fills group 0 and the first two words of group 1.
struct Raw6 {
  u32x6 g[2];
  RawScale s;
  template <bool FP6>
  __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, uint32_t blk, bool ok) {
    typedef unsigned int u32x6a __attribute__((ext_vector_type(6), aligned(8)));
    typedef unsigned int u32x2a __attribute__((ext_vector_type(2), aligned(8)));
    typedef __attribute__((address_space(1))) const u32x6a gu32x6a;  // global memory
    typedef __attribute__((address_space(1))) const u32x2a gu32x2a;
    const uint64_t b = ok ? blk : 0u;
    const uint64_t a0 = reinterpret_cast<uint64_t>(codes) + b * (FP6 ? 48 : 32);
    uint64_t a1 = a0 + 24;
    asm volatile("" : "+v"(a1));
    g[0] = *reinterpret_cast<gu32x6a*>(a0);
    if constexpr (FP6) {
      g[1] = *reinterpret_cast<gu32x6a*>(a1);
    } else {
      const u32x2a t = *reinterpret_cast<gu32x2a*>(a1);
      g[1] = u32x6{t.x, t.y, 0u, 0u, 0u, 0u};
    }
    s.load(scales, b, ok);
  }
  __device__ __forceinline__ uint32_t word(int i) const { return i < 6 ? g[0][i] : g[1][i - 6]; }
};
// FMTA: element format of the A operand (FP6, or E2M1 in MicroQonv+'s pair);
// FMTB: that of B, FP6.
template <int OP, int FMTA, int FMTB>
__global__ __launch_bounds__(256) void k_convs(const ConvParams p) {
  static_assert(Fmt<FMTB>::BITS == 6 && (FMTA == FMTB || FMTA == FMT_E2M1), "FP6 activations");
  constexpr bool MIXED = FMTA != FMTB;
  constexpr int MT = 256, NT = 256, WM = 2, KB = 4;
  constexpr int WTM = 128, WTN = 128, RM = 4, RN = 4;
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);
  constexpr int PL = 80;           // line pitch
  constexpr int PK = 576;          // k-row pitch
  constexpr int GK = 8 * PK + 64;  // the 8 k rows of one k-block + pad
  constexpr int SZL = 256 * PL, SZK = KB * GK;
  constexpr int A_SZ = A_ROWS ? SZL : SZK, B_SZ = B_ROWS ? SZL : SZK;
  constexpr int A_C = 0, B_C = A_SZ;
  constexpr int STAGE = A_SZ + B_SZ;
  constexpr int NST = 4;
  static_assert(STAGE % 16 == 0, "16-byte aligned stages");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE];
  using Raw = Raw6;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx<OP, MT, NT, KB> t;
  if (!t.init(p, tid)) return;
  const bool is_a = t.is_a;  // uniform per wave: the first two waves stage A

  // staging addresses of this thread's block: rows 0-3 from st0, rows 4-7
  // from st1, st_pitch apart.  Lines: row r is line 8 lblk + r (the swizzle
  // swaps the halves of line blocks with bit 1 set), at k-block kbl; k rows:
  // row r is k row 8 kbl + r, at column block lblk.
  const bool rows = is_a ? A_ROWS : B_ROWS;
  const int opbase = is_a ? A_C : B_C;
  const int sw = (t.lblk & 2) << 1;
  const int st0 = opbase + (rows ? (t.lblk * 8 + sw) * PL + t.kbl * 16 : t.kbl * GK + t.lblk * 16);
  const int st1 = rows ? opbase + (t.lblk * 8 + 4 - sw) * PL + t.kbl * 16 : st0 + 4 * PK;
  const int st_pitch = rows ? PL : PK;

  const uint8_t* my_codes = is_a ? p.a_codes : p.b_codes;
  const uint8_t* my_scales = is_a ? p.a_scales : p.b_scales;
  KWalk<OP, MT, NT, KB> walk;
  walk.init(p, t);
  uint32_t s_fetch = 0;  // k offset (s * KB) of the next fetch
  auto fetch = [&](Raw& g) {
    uint32_t blk;
    const bool ok = walk.next(s_fetch, blk);
    if (MIXED && is_a) g.template load<false>(my_codes, my_scales, blk, ok);
    else g.template load<true>(my_codes, my_scales, blk, ok);
    s_fetch += KB;
  };

  // Decode of the staged block into dw: 4 rows (a group) of 4 words of fp16
  // pairs, row-major.  A padding block (block 0's codes, scale code masked
  // to 0) converts to finite values (FP6 has no NaN or Inf code) that
  // mB = 0 turns into zeros.
  float sc;  // scale operand of the conversions (only its exponent is used)
  f16x2 m2;  // mantissa factor mB, twice
  uint32_t dw[16];
  auto set_scale = [&](const Raw& g) {
    const BlockScale bs(g.s.code());
    sc = bs.b;
    const _Float16 m = static_cast<_Float16>(bs.mb);
    m2 = f16x2{m, m};
  };
  // FP6 group G (rows 4G .. 4G+3) in one conversion
  auto convert_group = [&](const Raw& g, int G) {
    const auto v = [&] {
      if constexpr (FMTB == FMT_E3M2) return __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(g.g[G], sc);
      else return __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(g.g[G], sc);
    }();
    struct Words { uint32_t u[16]; };
    const Words wv = __builtin_bit_cast(Words, v);
#pragma unroll
    for (int k = 0; k < 16; ++k) dw[k] = wv.u[k];
  };
  // E2M1 row r (into dw row r % 4), two values per conversion
  auto convert_row = [&](const Raw& g, int r) {
    const uint32_t w = g.word(r);
    const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0);
    const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1);
    const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2);
    const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3);
    const int q = 4 * (r & 3);
    dw[q] = __builtin_bit_cast(uint32_t, v0);
    dw[q + 1] = __builtin_bit_cast(uint32_t, v1);
    dw[q + 2] = __builtin_bit_cast(uint32_t, v2);
    dw[q + 3] = __builtin_bit_cast(uint32_t, v3);
  };
  auto scale_words = [&](int k0) {
#pragma unroll
    for (int k = k0; k < k0 + 8; ++k) dw[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, dw[k]) * m2);
  };
  // rows r, r+1 of group G (r even, 0..2) of the decoded block into stage base
  auto write_rows = [&](uint8_t* base, int G, int r) {
    const int a = (G ? st1 : st0) + r * st_pitch;
    *reinterpret_cast<uint4*>(base + a) = make_uint4(dw[4 * r], dw[4 * r + 1], dw[4 * r + 2], dw[4 * r + 3]);
    *reinterpret_cast<uint4*>(base + a + st_pitch) =
        make_uint4(dw[4 * r + 4], dw[4 * r + 5], dw[4 * r + 6], dw[4 * r + 7]);
  };
  // Staging work of one step, as units placed after MFMAs: FP6 units K =
  // 0..11 after MFMA 8 + K, E2M1 units K = 0..17 after MFMA K.  The block's
  // set is refilled (fetch) after the last unit that reads it (both after
  // MFMA 15).  In MicroQonv+'s pair the A-staging waves run the E2M1 units
  // and the B-staging waves the FP6 units (a wave-uniform branch per slot).
  auto stage_fp6 = [&]<int K>(Raw& g, uint8_t* wr) {
    if constexpr (K == 0) set_scale(g);
    else if constexpr (K == 1 || K == 6) convert_group(g, K == 6);
    else if constexpr (K == 2 || K == 8) scale_words(0);
    else if constexpr (K == 3 || K == 9) scale_words(8);
    else if constexpr (K == 4 || K == 10) write_rows(wr, K == 10, 0);
    else if constexpr (K == 5 || K == 11) write_rows(wr, K == 11, 2);
    else if constexpr (K == 7) fetch(g);
  };
  // rows 2P, 2P+1 in units 1 + 4P .. 4 + 4P (the last pair: 13, 14, then
  // the refill, 16, 17)
  auto stage_e2m1 = [&]<int K>(Raw& g, uint8_t* wr) {
    if constexpr (K == 0) set_scale(g);
    else if constexpr (K == 15) fetch(g);
    else {
      constexpr int P = K < 15 ? (K - 1) / 4 : 3, U = K < 15 ? (K - 1) % 4 : K - 14;
      if constexpr (U == 0 || U == 1) convert_row(g, 2 * P + U);
      else if constexpr (U == 2) scale_words(8 * (P & 1));
      else write_rows(wr, P >> 1, 2 * (P & 1));
    }
  };
  auto stage_slot = [&]<int M>(Raw& g, uint8_t* wr) {
    constexpr bool F = M >= 8 && M < 20, E = M < 18;
    if constexpr (!MIXED) {
      if constexpr (F) stage_fp6.template operator()<M - 8>(g, wr);
    } else if constexpr (F && E) {
      if (is_a) stage_e2m1.template operator()<M>(g, wr);
      else stage_fp6.template operator()<M - 8>(g, wr);
    } else if constexpr (E) {
      if (is_a) stage_e2m1.template operator()<M>(g, wr);
    } else if constexpr (F) {
      if (!is_a) stage_fp6.template operator()<M - 8>(g, wr);
    }
  };
  auto stage_block = [&](Raw& g, uint8_t* base) {
    set_scale(g);
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      if (MIXED && is_a) {
#pragma unroll
        for (int r = 0; r < 4; ++r) convert_row(g, 4 * G + r);
      } else {
        convert_group(g, G);
      }
      scale_words(0);
      scale_words(8);
      write_rows(base, G, 0);
      write_rows(base, G, 2);
    }
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment read offsets (slice 0; slice 1 is 32 bytes further for lines,
  // 2 GK for k rows).  Lines: line wX*128 + i*32 + lane%32 (swizzled), K
  // half lane/32; fragment i adds 32 lines.  K rows: the lane supplies row
  // e = (lane%16)/4 (and 4 + e) of k-block lane/32, columns 4 (lane%4) ..
  // +3 of the 16-column group (lane/16)%2; fragment i adds 32 columns.
  const int l32 = lane & 31, half = lane >> 5;
  const int line_off = (l32 ^ ((l32 >> 2) & 4)) * PL + half * 16;
  const int krow_off = half * GK + ((lane & 15) >> 2) * PK + (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
  const int a_frag = A_C + (A_ROWS ? wm * 128 * PL + line_off : wm * 256 + krow_off);
  const int b_frag = B_C + (B_ROWS ? wn * 128 * PL + line_off : wn * 256 + krow_off);
  auto read_frag = [&](const uint8_t* q, bool line) -> f16x8 {
    if (line) return *reinterpret_cast<const f16x8*>(q);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * PK));
    return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // fragment i of A (j of B) of slice `slice` of the stage at `base`
  auto frag_a = [&](const uint8_t* base, int slice, int i) {
    return read_frag(base + a_frag + (A_ROWS ? i * 32 * PL + slice * 32 : i * 64 + slice * 2 * GK), A_ROWS);
  };
  auto frag_b = [&](const uint8_t* base, int slice, int j) {
    return read_frag(base + b_frag + (B_ROWS ? j * 32 * PL + slice * 32 : j * 64 + slice * 2 * GK), B_ROWS);
  };
  f16x8 fa0[RM], fb0[RN], fa1[RM], fb1[RN];  // fragments of slice 0 and slice 1

  // One step (its fragments of both slices in fa0/fb0 and fa1/fb1): MFMA M
  // (slice M / 16, column (M % 16) / 4, row M % 4) is followed by its work
  // and a scheduling barrier (a wave hides only a few VALU operations and
  // LDS accesses behind each MFMA): after MFMAs 20-27 the slice-0 fragments
  // of the next stage (nxt), and the slice-1 fragments of nxt each right
  // after the last MFMA that reads its register (B column j after MFMA
  // 19 + 4j, A row i after MFMA 28 + i), so that a stage is read only in
  // the step before its own; and the staging units of the block in G into
  // the stage at wr, which refill G two steps ahead.  A barrier at the end
  // where BAR is set.
  auto slot = [&]<int M, int BAR>(Raw& G, const uint8_t* nxt, uint8_t* wr) {
    constexpr int i = M % 4, j = (M % 16) / 4;
    if constexpr (M < 16)
      acc[i][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa0[i]), reinterpret_cast<const uint16_t*>(&fb0[j]), acc[i][j]);
    else
      acc[i][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa1[i]), reinterpret_cast<const uint16_t*>(&fb1[j]), acc[i][j]);
    if constexpr (M >= 20 && M < 28) {
      if constexpr (M % 2 == 0) fa0[(M - 20) / 2] = frag_a(nxt, 0, (M - 20) / 2);
      else fb0[(M - 20) / 2] = frag_b(nxt, 0, (M - 20) / 2);
    }
    if constexpr (M == 19 || M == 23 || M == 27 || M == 31) fb1[(M - 19) / 4] = frag_b(nxt, 1, (M - 19) / 4);
    if constexpr (M >= 28) fa1[M - 28] = frag_a(nxt, 1, M - 28);
    stage_slot.template operator()<M>(G, wr);
    if constexpr (M == 31 && BAR) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](Raw& G, const uint8_t* nxt, uint8_t* wr, auto bar_c) {
    [&]<int... M>(std::integer_sequence<int, M...>) {
      (slot.template operator()<M, decltype(bar_c)::value>(G, nxt, wr), ...);
    }(std::make_integer_sequence<int, 32>());
  };

  const int nsteps = (t.kb_end - t.kb_begin + KB - 1) / KB;
  if (nsteps > 0) {
    Raw g0, g1;  // the blocks that even and odd steps stage
    fetch(g0);
    fetch(g1);
    stage_block(g0, lds);
    stage_block(g1, lds + STAGE);
    fetch(g0);
    stage_block(g0, lds + 2 * STAGE);
    fetch(g0);
    fetch(g1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      fa0[i] = frag_a(lds, 0, i);
      fa1[i] = frag_a(lds, 1, i);
    }
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      fb0[j] = frag_b(lds, 0, j);
      fb1[j] = frag_b(lds, 1, j);
    }
    // Step s computes stage s % 4 (its fragments read in step s - 1), reads
    // stage (s + 1) % 4 and stages the block of step s + 3 into stage
    // (s + 3) % 4 from register set s % 2, which it then refills with the
    // block of step s + 5.  A barrier ends every even step only: a stage
    // written in step s is read in step s + 2, and the one it overwrites was
    // last read in step s - 2, so a barrier at the end of s or s + 1, and one
    // at the end of s - 2 or s - 1, orders both.  One loop iteration runs the
    // four steps of the pattern, so every stage offset is an immediate of its
    // LDS instruction.  The step count is rounded up to a multiple of four;
    // the extra steps see padding blocks only (zero values: they add exact
    // zeros).
    for (int s = 0; s < nsteps; s += 4) {
      step(g0, lds + STAGE, lds + 3 * STAGE, IC<1>{});
      step(g1, lds + 2 * STAGE, lds, IC<0>{});
      step(g0, lds + 3 * STAGE, lds + STAGE, IC<1>{});
      step(g1, lds, lds + 2 * STAGE, IC<0>{});
    }
  }
  store_tile<OP, MT, NT, KB, WTM, WTN, RM, RN>(p, t, acc, lane, wm, wn);
}

template <int FMTA, int FMTB>
void launch_fmt_staged(int op, const ConvParams& p, dim3 grid, hipStream_t s) {
  switch (op) {
    case OP_FWD: hipLaunchKernelGGL((k_convs<OP_FWD, FMTA, FMTB>), grid, dim3(256), 0, s, p); break;
    case OP_DGRAD:
      if constexpr (FMTA == FMTB) hipLaunchKernelGGL((k_convs<OP_DGRAD, FMTA, FMTB>), grid, dim3(256), 0, s, p);
      break;
    default: hipLaunchKernelGGL((k_convs<OP_WGRAD, FMTA, FMTB>), grid, dim3(256), 0, s, p); break;
  }
}

}  // namespace

namespace gemm {

// The 256x256 kernel of FP6 activations; false (nothing launched) for a
// format pair it does not take (FP6 throughout; E2M1 with FP6 activations in
// the forward and weight-gradient GEMMs) or where its K walk needs the
// division-based block search (an innermost K extent below 4 k-blocks).
bool launch_staged(int op, int fmt_a, int fmt_b, const ConvParams& p, dim3 grid, hipStream_t s) {
  if (!kwalk_ok(op, p, 4)) return false;
  if (fmt_a == fmt_b) {
    if (fmt_a == FMT_E2M3) launch_fmt_staged<FMT_E2M3, FMT_E2M3>(op, p, grid, s);
    else if (fmt_a == FMT_E3M2) launch_fmt_staged<FMT_E3M2, FMT_E3M2>(op, p, grid, s);
    else return false;
    return true;
  }
  if (fmt_a != FMT_E2M1 || op == OP_DGRAD) return false;
  if (fmt_b == FMT_E3M2) launch_fmt_staged<FMT_E2M1, FMT_E3M2>(op, p, grid, s);
  else if (fmt_b == FMT_E2M3) launch_fmt_staged<FMT_E2M1, FMT_E2M3>(op, p, grid, s);
  else return false;
  return true;
}

}  // namespace gemm
}  // namespace mx
