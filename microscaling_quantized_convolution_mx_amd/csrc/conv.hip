// Convolution GEMMs on microscaled operands: the E2M1 kernels that keep the
// 4-bit codes in LDS and decode them at fragment read, the weight-gradient
// split reduction, tile selection and the launchers behind the C ABI
// (MicroQonv, arXiv 2609.28358, §IV-B).  The generic kernel and the GEMM
// formulation are in conv_kernels.h.
#include "conv_kernels.h"

namespace mx {
namespace {


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

// Half h (values 4h..4h+3) of decode_frag, for placing between MFMAs.
__device__ __forceinline__ void decode_half(f16x8& f, uint32_t codes, uint32_t sw, int h) {
  const float sc = __uint_as_float(sw);
  // the mantissa factor in both halves: a splat of the low half, which the
  // packed multiply takes through its operand select (no extra instruction)
  const f16x2 sw2 = __builtin_bit_cast(f16x2, sw);
  const f16x2 m2 = {sw2[0], sw2[0]};
  if (h == 0) {
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 0) * m2;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 1) * m2;
    f[0] = p0[0]; f[1] = p0[1]; f[2] = p1[0]; f[3] = p1[1];
  } else {
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 2) * m2;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc, 3) * m2;
    f[4] = p2[0]; f[5] = p2[1]; f[6] = p3[0]; f[7] = p3[1];
  }
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
  // Where the A/B staging split falls inside a wave (MT < 128) and A and B
  // are staged differently (fwd), that wave runs both sides of the
  // transpose branch in stage_block; nothing else depends on the split.
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
  const bool rows = is_a ? A_ROWS : B_ROWS;

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

// E2M1, 256x256 tile, 4 waves of 128x128, one workgroup per CU (the 256
// accumulator registers of a wave fill the AGPR file).  LDS holds the raw
// 4-bit codes of four K steps; each wave decodes its MFMA fragments from
// them (conversion with the block scale's exponent, then a packed multiply
// by its mantissa factor: exact in fp16).
//
// A wave hides VALU work behind its own MFMAs only a few operations at a
// time (on this GPU about 4 VALU operations per 32x32x16 MFMA; past that
// every operation adds its issue time), so each fragment is decoded in the
// column before the one that uses it, in halves placed after single MFMAs,
// and the raw fragments of the next stage are read a whole step ahead into
// a second register set.
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
// unrolled twice so that the register sets are static (the stage offsets
// rotate at run time).
template <int OP>
__global__ __launch_bounds__(256) void k_conv4w(const ConvParams p) {
  constexpr int MT = 256, NT = 256, WM = 2, KB = 4;
  constexpr int WTM = 128, WTN = 128, RM = 4, RN = 4;
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);
  constexpr int PITCH = 136, OPND = 32 * PITCH, SCL = 32 * 16;
  constexpr int A_C = 0, B_C = OPND, A_S = 2 * OPND, B_S = 2 * OPND + SCL;
  constexpr int STAGE = 2 * OPND + 2 * SCL;
  constexpr int NST = 4;
  constexpr int LUT = NST * STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE + 1024];

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
      for (int r = r0; r < r0 + 2; ++r)
        *reinterpret_cast<uint32_t*>(base + st_code + r * (A_ROWS ? 16 : PITCH)) = g.w[r];
    } else {
      if (__builtin_amdgcn_readfirstlane(static_cast<int>(rows))) {
#pragma unroll
        for (int r = r0; r < r0 + 2; ++r) *reinterpret_cast<uint32_t*>(base + st_code + r * 16) = g.w[r];
      } else {
#pragma unroll
        for (int r = r0; r < r0 + 2; ++r) *reinterpret_cast<uint32_t*>(base + st_code + r * PITCH) = g.w[r];
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
  u32x2 ra[2][RM], sa[2][RM], rb[2][RN], sbv[2][RN];  // raw fragments of two stages (.x slice 0, .y slice 1)
  auto read_code = [&](const uint8_t* q, bool line) -> u32x2 {
    if (line) return *reinterpret_cast<const u32x2*>(q);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2*)(q)));
  };
  // part q (0..3) of the raw fragments of a stage: A and B fragment q with
  // their scale words
  auto read_raw = [&](auto set_c, const uint8_t* base, int q) {
    constexpr int Q = decltype(set_c)::value;
    ra[Q][q] = read_code(base + a_code + q * (A_ROWS ? 4 * PITCH : 16), A_ROWS);
    sa[Q][q] = *reinterpret_cast<const u32x2*>(base + a_scale + q * 64);
    rb[Q][q] = read_code(base + b_code + q * (B_ROWS ? 4 * PITCH : 16), B_ROWS);
    sbv[Q][q] = *reinterpret_cast<const u32x2*>(base + b_scale + q * 64);
  };
  f16x8 fa0[RM], fa1[RM];  // A fragments of slice 0 and slice 1

  // One column j of a slice: MFMA i is followed by work unit i (a few VALU
  // operations and LDS accesses), each closed by a scheduling barrier, so
  // that the wave issues the decode work between MFMAs instead of in runs.
  auto column = [&](const f16x8 (&fa)[RM], const f16x8& fb, int j, auto&& u0, auto&& u1, auto&& u2, auto&& u3) {
    acc[0][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa[0]), reinterpret_cast<const uint16_t*>(&fb), acc[0][j]);
    u0();
    __builtin_amdgcn_sched_barrier(0);
    acc[1][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa[1]), reinterpret_cast<const uint16_t*>(&fb), acc[1][j]);
    u1();
    __builtin_amdgcn_sched_barrier(0);
    acc[2][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa[2]), reinterpret_cast<const uint16_t*>(&fb), acc[2][j]);
    u2();
    __builtin_amdgcn_sched_barrier(0);
    acc[3][j] = mfma32<true>(reinterpret_cast<const uint16_t*>(&fa[3]), reinterpret_cast<const uint16_t*>(&fb), acc[3][j]);
    u3();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Step s on stage s%4 (raw fragments in set P; slice-0 A fragments and the
  // slice-0 column-0 B fragment fbc decoded).  Every fragment is decoded in
  // the column before the one that uses it, in halves after single MFMAs:
  // slice 0 decodes the slice-1 A fragments and the next B fragment; slice 1
  // the next B fragment and the next step's slice-0 A fragments (set Q,
  // read from stage (s+1)%4 during slice-0 column 0).  The block in G is
  // staged into stage wr_c and G refilled two steps ahead; a barrier at the
  // end where bar_c is set.  Stage offsets are compile-time constants.
  f16x8 fbc;
  auto step = [&](auto set_c, RawBlock<FMT_E2M1>& G, auto nxt_c, auto wr_c, auto bar_c) {
    constexpr int P = decltype(set_c)::value, Q = P ^ 1;
    uint8_t* wbase = lds + decltype(wr_c)::value;
    const uint8_t* nbase = lds + decltype(nxt_c)::value;
    f16x8 fbA, fbB;
    // slice 0
    column(fa0, fbc, 0,
           [&] { read_raw(IC<Q>{}, nbase, 0); decode_half(fa1[0], ra[P][0].y, sa[P][0].y, 0); },
           [&] { read_raw(IC<Q>{}, nbase, 1); decode_half(fa1[0], ra[P][0].y, sa[P][0].y, 1); },
           [&] { read_raw(IC<Q>{}, nbase, 2); decode_half(fbA, rb[P][1].x, sbv[P][1].x, 0); },
           [&] { read_raw(IC<Q>{}, nbase, 3); decode_half(fbA, rb[P][1].x, sbv[P][1].x, 1); });
    column(fa0, fbA, 1,
           [&] { lookup_scale(G); decode_half(fa1[1], ra[P][1].y, sa[P][1].y, 0); },
           [&] { write_rows(G, wbase, 0); decode_half(fa1[1], ra[P][1].y, sa[P][1].y, 1); },
           [&] { write_rows(G, wbase, 2); decode_half(fbB, rb[P][2].x, sbv[P][2].x, 0); },
           [&] { write_rows(G, wbase, 4); decode_half(fbB, rb[P][2].x, sbv[P][2].x, 1); });
    column(fa0, fbB, 2,
           [&] { write_rows(G, wbase, 6); decode_half(fa1[2], ra[P][2].y, sa[P][2].y, 0); },
           [&] { fetch(G); decode_half(fa1[2], ra[P][2].y, sa[P][2].y, 1); },
           [&] { *reinterpret_cast<uint32_t*>(wbase + st_scale) = sws; decode_half(fbA, rb[P][3].x, sbv[P][3].x, 0); },
           [&] { decode_half(fbA, rb[P][3].x, sbv[P][3].x, 1); });
    column(fa0, fbA, 3,
           [&] { decode_half(fa1[3], ra[P][3].y, sa[P][3].y, 0); },
           [&] { decode_half(fa1[3], ra[P][3].y, sa[P][3].y, 1); },
           [&] { decode_half(fbB, rb[P][0].y, sbv[P][0].y, 0); },
           [&] { decode_half(fbB, rb[P][0].y, sbv[P][0].y, 1); });
    // slice 1 (fa0 is free: it takes the next step's slice-0 A fragments)
    column(fa1, fbB, 0,
           [&] { decode_half(fbA, rb[P][1].y, sbv[P][1].y, 0); },
           [&] { decode_half(fbA, rb[P][1].y, sbv[P][1].y, 1); },
           [&] { decode_half(fa0[0], ra[Q][0].x, sa[Q][0].x, 0); },
           [&] { decode_half(fa0[0], ra[Q][0].x, sa[Q][0].x, 1); });
    column(fa1, fbA, 1,
           [&] { decode_half(fbB, rb[P][2].y, sbv[P][2].y, 0); },
           [&] { decode_half(fbB, rb[P][2].y, sbv[P][2].y, 1); },
           [&] { decode_half(fa0[1], ra[Q][1].x, sa[Q][1].x, 0); },
           [&] { decode_half(fa0[1], ra[Q][1].x, sa[Q][1].x, 1); });
    column(fa1, fbB, 2,
           [&] { decode_half(fbA, rb[P][3].y, sbv[P][3].y, 0); },
           [&] { decode_half(fbA, rb[P][3].y, sbv[P][3].y, 1); },
           [&] { decode_half(fa0[2], ra[Q][2].x, sa[Q][2].x, 0); },
           [&] { decode_half(fa0[2], ra[Q][2].x, sa[Q][2].x, 1); });
    column(fa1, fbA, 3,
           [&] { decode_half(fa0[3], ra[Q][3].x, sa[Q][3].x, 0); },
           [&] { decode_half(fa0[3], ra[Q][3].x, sa[Q][3].x, 1); },
           [&] { decode_half(fbc, rb[Q][0].x, sbv[Q][0].x, 0); },
           [&] {
             decode_half(fbc, rb[Q][0].x, sbv[Q][0].x, 1);
             if constexpr (decltype(bar_c)::value) __syncthreads();
           });
  };

  const int nsteps = (t.kb_end - t.kb_begin + KB - 1) / KB;
  if (nsteps > 0) {
    RawBlock<FMT_E2M1> g0, g1;  // the blocks that even and odd steps stage
    auto stage_block = [&](const RawBlock<FMT_E2M1>& g, uint8_t* base) {
      lookup_scale(g);
      write_rows(g, base, 0);
      write_rows(g, base, 2);
      write_rows(g, base, 4);
      write_rows(g, base, 6);
      *reinterpret_cast<uint32_t*>(base + st_scale) = sws;
    };
    fetch(g0);
    fetch(g1);
    __syncthreads();  // scale-word table
    stage_block(g0, lds);
    stage_block(g1, lds + STAGE);
    fetch(g0);
    stage_block(g0, lds + 2 * STAGE);
    fetch(g0);
    fetch(g1);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) read_raw(IC<0>{}, lds, q);
#pragma unroll
    for (int i = 0; i < RM; ++i) fa0[i] = decode_frag(ra[0][i].x, sa[0][i].x);
    fbc = decode_frag(rb[0][0].x, sbv[0][0].x);
    // Step s computes from stage s % 4, reads stage (s + 1) % 4 (all of its
    // raw fragments) and stages the block of step s + 3 into stage
    // (s + 3) % 4 from register set s % 2, which it then refills with the
    // block of step s + 5.  A barrier ends every even step only: a stage
    // written in step s is read in step s + 2, and the one it overwrites was
    // last read in step s - 2, so a barrier at the end of s or s + 1, and one
    // at the end of s - 2 or s - 1, orders both.  One loop iteration runs the
    // four steps of the pattern, so every stage offset is an immediate of its
    // LDS instruction (no address arithmetic per step).  The step count is
    // rounded up to a multiple of four; the extra steps see padding blocks
    // only (zero scale words: they add exact zeros).
    for (int s = 0; s < nsteps; s += 4) {
      step(IC<0>{}, g0, IC<STAGE>{}, IC<3 * STAGE>{}, IC<1>{});
      step(IC<1>{}, g1, IC<2 * STAGE>{}, IC<0>{}, IC<0>{});
      step(IC<0>{}, g0, IC<3 * STAGE>{}, IC<STAGE>{}, IC<1>{});
      step(IC<1>{}, g1, IC<0>{}, IC<2 * STAGE>{}, IC<0>{});
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

Tile pick_tile(int64_t M, int64_t ncols, int64_t zdim) {
  const int cap = mt_cap(M);
  Tile best = {0, 0, 0, 0, 0};
  int64_t best_reach = -1;
  for (const Tile& t : kTiles) {
    if (t.mt > cap) continue;
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
Tile pick_wgrad_tile(int64_t M, int64_t ncols) {
  const int cap = mt_cap(M);
  double best_eff = 0.0;
  for (const Tile& t : kTiles) {
    if (t.mt > cap) continue;
    const double eff = static_cast<double>(M * ncols) /
                       (static_cast<double>((M + t.mt - 1) / t.mt * t.mt) * ((ncols + t.nt - 1) / t.nt * t.nt));
    if (eff > best_eff) best_eff = eff;
  }
  for (const Tile& t : kTiles) {
    if (t.mt > cap) continue;
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
    if (t.mt == 64 && t.nt == 256) return launch_tile4<OP, 64, 256, 1, 4>(p, grid, s);
    if (t.mt == 32 && t.nt == 256) return launch_tile4<OP, 32, 256, 1, 4>(p, grid, s);
  } else if constexpr (FMT == FMT_E4M3) {
    // E4M3 on the 256x256 tile: byte codes in LDS, decoded at fragment read
    if (t.mt == 256 && t.nt == 256 && launch_conv8(OP, p, grid, s)) return;
  } else if constexpr (FMT == FMT_E2M3) {
    // E2M3 on the 256x256 tile: fetched two K steps ahead, fp16 in LDS
    if (t.mt == 256 && t.nt == 256 && launch_staged(OP, FMT_E2M3, FMT_E2M3, p, grid, s)) return;
  }
  launch_generic<OP, FMT, FMT>(p, t, grid, s);
}

template <int OP>
bool launch_op(const ConvParams& p, int fmt_a, int fmt_b, const Tile& t, dim3 grid, hipStream_t s) {
  if (fmt_a == fmt_b) {
    switch (fmt_a) {
      case FMT_E2M1: launch_fmt<OP, FMT_E2M1>(p, t, grid, s); return true;
      case FMT_E2M3: launch_fmt<OP, FMT_E2M3>(p, t, grid, s); return true;
      case FMT_E4M3: launch_fmt<OP, FMT_E4M3>(p, t, grid, s); return true;
      default: break;
    }
  }
  return launch_mixed(OP, p, fmt_a, fmt_b, t, grid, s);
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
  Tile t = pick_wgrad_tile(g.c_out, ncol);
  // all-E2M1 128x256, 64x256 and 32x256 tiles run k_conv4 (decode at fragment read,
  // K steps of 4 k-blocks, two workgroups per CU); p.ks_split counts its steps
  const bool decode_tile = g.fmt == FMT_E2M1 && g.afmt == FMT_E2M1 && t.mt <= 128 && t.nt == 256;
  if (decode_tile) t.kb = 4;
  const int64_t ksteps = (kb_total + t.kb - 1) / t.kb;
  const int64_t tiles = ((g.c_out + t.mt - 1) / t.mt) * ((ncol + t.nt - 1) / t.nt);
  // About one round of workgroups: 1024 waves, or 2048 for the 128- and
  // 64-row k_conv4 tiles, which run two workgroups per CU.  More splits
  // shorten each K loop but add partials to write and reduce (sweeps over
  // the ResNet stacks put the optimum there; the 32-row tile of ResNet-32's
  // 16- and 32-channel layers does better with 1024).  Rounded down: a last,
  // nearly empty round of workgroups costs a full one.
  const int64_t target_waves = decode_tile && t.mt >= 64 ? 2048 : 1024;
  int64_t splits = (target_waves / t.waves) / tiles;
  const int64_t max_by_k = ksteps / 4;
  if (splits > max_by_k) splits = max_by_k;
  if (splits < 1) splits = 1;
  if (splits > 65535) splits = 65535;
  return {t, static_cast<int>(splits)};
}

// Weight gradient on E8M0 32x32 blocks: K steps of 128, about one round of
// workgroups with at least 4 K steps per split.
// E8M0 GEMM tile.  The 256x256 tile (one workgroup per CU) reuses each
// operand block most; the 128x128 tile runs two workgroups per CU, so one
// workgroup's barrier and load waits are covered by the other's MFMAs, and
// wastes less on 64- and 128-row GEMMs.  256 only where M > 128 and the
// launch still has about four workgroups per CU (fwd, dgrad: zdim = stride
// phases), or for the weight gradient (zdim = K steps) one full round with
// the largest K split.
int mx_tile(int op, int64_t M, int64_t ncols, int64_t zdim) {
  if (M <= 128) return 128;
  const int64_t tiles256 = ((M + 255) / 256) * ((ncols + 255) / 256);
  if (op == OP_WGRAD) return tiles256 * (zdim / 4) >= 256 ? 256 : 128;
  return tiles256 * zdim >= 1024 ? 256 : 128;
}

WgradPlan wgrad_plan_mx(const Geom& g) {
  const int64_t ksteps = (static_cast<int64_t>(g.ho) * g.wo * (g.n / 32) + kMxStepBlocks - 1) / kMxStepBlocks;
  const int T = mx_tile(OP_WGRAD, g.c_out, static_cast<int64_t>(g.k_h) * g.k_w * g.c_in, ksteps);
  const int64_t ncol = static_cast<int64_t>(g.k_h) * g.k_w * g.c_in;
  const int64_t tiles = ((g.c_out + T - 1) / T) * ((ncol + T - 1) / T);
  // about one round of workgroups: one per CU for the 256 tile, two for 128
  int64_t splits = (T == 256 ? 256 : 512) / tiles;
  if (splits > ksteps / 4) splits = ksteps / 4;
  if (splits < 1) splits = 1;
  if (splits > 65535) splits = 65535;
  return {Tile{T, T, 2, 4, 4}, static_cast<int>(splits)};
}

// Band order of a fwd / dgrad launch's column tiles (TileCtx::init): rows
// of `row_pos` output positions, `rows` of them, each a whole number of
// NT-column tiles; bands of 4 rows.
void set_band(ConvParams& p, int rows, int row_pos, int nt) {
  const int64_t cb_per_row = static_cast<int64_t>(row_pos) * p.nb;
  const int tile_cb = nt / 8;
  if (rows >= 8 && cb_per_row % tile_cb == 0) {
    p.band_tpr = static_cast<int32_t>(cb_per_row / tile_cb);
    p.band_rows = 4;
  }
}

// Forward launch geometry: tile, grid and waves per workgroup.
struct FwdPlan {
  Tile t;
  dim3 grid;
};
FwdPlan fwd_plan(const Geom& g, const ConvParams& p) {
  const Tile t = pick_tile(p.M, static_cast<int64_t>(p.ncb) * 8, 1);
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
  p.stream_out = static_cast<int64_t>(g.ho) * g.wo * g.c_out * g.n * 4 > static_cast<int64_t>(kStreamOutBytes);
  p.amax_out = reinterpret_cast<uint32_t*>(y_amax);
  int64_t nslots = 0;
  if (g.block == 32) {
    const int T = mx_tile(OP_FWD, p.M, static_cast<int64_t>(p.ncb) * 8, 1);
    if (p.ncb > 0) launch_mx(OP_FWD, T, p, dim3((p.ncb * 8 + T - 1) / T, (p.M + T - 1) / T, 1), s);
    return hipGetLastError();
  }
  if (p.ncb > 0) {
    const FwdPlan pl = fwd_plan(g, p);
    nslots = static_cast<int64_t>(pl.grid.x) * pl.grid.y * pl.grid.z * pl.t.waves;
    set_band(p, g.ho, g.wo, pl.t.nt);
    if (!launch_op<OP_FWD>(p, g.fmt, g.afmt, pl.t, pl.grid, s)) return hipErrorNotSupported;
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
  p.stream_out = static_cast<int64_t>(g.h) * g.w * g.c_in * g.n * 4 > static_cast<int64_t>(kStreamOutBytes);
  if (p.ncb == 0) return hipSuccess;
  if (g.block == 32) {
    const int T = mx_tile(OP_DGRAD, p.M, static_cast<int64_t>(p.ncb) * 8, g.sh * g.sw);
    launch_mx(OP_DGRAD, T, p, dim3((p.ncb * 8 + T - 1) / T, (p.M + T - 1) / T, g.sh * g.sw), s);
    return hipGetLastError();
  }
  const Tile t = pick_tile(p.M, static_cast<int64_t>(p.ncb) * 8, g.sh * g.sw);
  dim3 grid((p.ncb * 8 + t.nt - 1) / t.nt, (p.M + t.mt - 1) / t.mt, g.sh * g.sw);
  if (g.sh == 1 && g.sw == 1) set_band(p, g.h, g.w, t.nt);  // one phase: the positions are (h, w)
  if (!launch_op<OP_DGRAD>(p, g.fmt, g.fmt, t, grid, s)) return hipErrorNotSupported;
  return hipGetLastError();
}

size_t wgrad_workspace_bytes(const Geom& g) {
  const WgradPlan pl = g.block == 32 ? wgrad_plan_mx(g) : wgrad_plan(g);
  return static_cast<size_t>(pl.splits) * g.c_out * g.k_h * g.k_w * g.c_in * sizeof(float);
}

hipError_t launch_conv_wgrad(const Geom& g, const mx_qtensor* dyq, const mx_qtensor* xq, float* dw,
                             void* workspace, hipStream_t s) {
  ConvParams p = base_params(g);
  const bool mxb = g.block == 32;
  const WgradPlan pl = mxb ? wgrad_plan_mx(g) : wgrad_plan(g);
  p.M = g.c_out;
  p.ncol = g.k_h * g.k_w * g.c_in;
  p.ncb = p.ncol / 8;
  p.kb_total = g.ho * g.wo * (g.n / 8);
  // K steps: of the tile's KB 8-blocks, or of kMxStepBlocks 32-blocks
  const int ksteps = mxb ? (g.ho * g.wo * (g.n / 32) + kMxStepBlocks - 1) / kMxStepBlocks
                         : (p.kb_total + pl.t.kb - 1) / pl.t.kb;
  p.ks_split = (ksteps + pl.splits - 1) / pl.splits;
  p.a_codes = static_cast<const uint8_t*>(dyq->codes); p.a_scales = dyq->scales; p.a_t = dyq->tensor_scale;
  p.b_codes = static_cast<const uint8_t*>(xq->codes); p.b_scales = xq->scales; p.b_t = xq->tensor_scale;
  p.out = static_cast<float*>(workspace);
  dim3 grid((p.ncol + pl.t.nt - 1) / pl.t.nt, (p.M + pl.t.mt - 1) / pl.t.mt, pl.splits);
  if (mxb) launch_mx(OP_WGRAD, pl.t.mt, p, grid, s);
  else if (!launch_op<OP_WGRAD>(p, g.fmt, g.afmt, pl.t, grid, s)) return hipErrorNotSupported;
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
