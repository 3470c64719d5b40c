// Convolution GEMMs for E4M3 elements with the codes kept in LDS as bytes
// and decoded at fragment read (MicroQonv, arXiv 2609.28358, §IV-B; FP8
// elements of §IV-E and §VI-B).
//
// The generic kernel (conv_kernels.h) decodes every staged E4M3 block into
// bf16 K-lines (an fp32 conversion and product per element), so its LDS
// carries two bytes per element in and out and its staging threads spend
// 16 operations per 8 values.  Here LDS holds the E4M3 codes as they are and
// every wave decodes its own MFMA fragments between its MFMAs, like the E2M1
// kernel in conv.hip:
//   v_cvt_scalef32_pk_f16_fp8 applies the exponent of the scale word (the
//   block scale's, lowered by 2^-2), a packed fp16 multiply its mantissa
//   factor mB = B / 2^floor(log2 B).
// Both steps are exact, so the fp16 MFMA sums the exact products of Eq. 7
// scaled by 2^-4, which the epilogue undoes exactly:
//   - every E4M3 value, element g or block scale B, is a multiple of 2^-9
//     with at most 4 significant bits, so g * B * 2^-2 is a multiple of 2^-20
//     with at most 8 significant bits and at most 448 * 448 / 4 = 50176:
//     an fp16 value (a subnormal below 2^-14); so is the conversion's
//     intermediate g * 2^(floor(log2 B) - 2);
//   - without the lowering the largest values (up to 200704) would overflow
//     fp16;
//   - gfx950's conversion and packed multiply produce fp16 subnormals
//     exactly (checked on the GPU for every E4M3 code at every scale
//     exponent from 2^-11 to 2^0: no difference from the exact values).
//
// Tile: 256x256, 4 waves of 128x128 (one workgroup per CU: a wave's 16
// accumulator tiles fill its 256 AGPRs), K steps of 4 k-blocks (32 K values:
// two 16-wide MFMA slices), four LDS stages, block fetches two steps ahead.
// As in the E2M1 kernel, every fragment is decoded in the column before
// the one that uses it, in halves placed after single MFMAs (a wave hides
// only about 4 VALU operations behind each MFMA), and the raw fragments of
// the next stage are read a whole step ahead into a second register set.
// Stage layout, per operand:
//   block rows along M/N (fwd A, wgrad A and B): 32 line blocks of 8 lines
//     of 32 bytes (the 4 k-blocks of a row in the order 0, 2, 1, 3, so that
//     lane half h reads k-blocks h and 2+h -- its K slots of slice 0 and
//     slice 1 -- with one 16-byte read), pitch 304 bytes;
//   block rows along K (fwd B, dgrad A and B): 32 k rows of 256 codes,
//     the rows of k-block kb at rows 8 * slot(kb), pitch 272 bytes plus
//     16 after every 8 rows; the transposing LDS read (an 8 x 16 byte
//     transpose within each group of 16 lanes, rows from lane pairs) turns
//     8 k rows into the k-runs of 16 columns;
//   scale words: one per line block and k-block (same slot order), from a
//     256-entry table (entry 0 is 0, which also masks padding blocks).
#include "conv_kernels.h"

namespace mx {
namespace {

typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2v;

// exponent lowering of the decode (keeps 448 * 448 below the fp16 maximum)
constexpr int kShift = 2;

// Scale word of an E4M3 block scale code: the fp32 exponent field of B
// lowered by sh | the fp16 mantissa factor mB in the low 16 bits; 0 for a
// zero scale.  The conversions use only the exponent of their scale operand.
__device__ __forceinline__ uint32_t scale_word8(uint32_t code, int sh) {
  const float b = code_value<ScaleFmt>(code);
  const uint32_t bits = __float_as_uint(b);
  const _Float16 mb = static_cast<_Float16>(__uint_as_float((bits & 0x007FFFFFu) | 0x3F800000u));
  return code == 0u ? 0u
                    : ((bits & 0x7F800000u) - (static_cast<uint32_t>(sh) << 23)) | __builtin_bit_cast(uint16_t, mb);
}

// Eight fp16 values g * B * 2^-kShift of one fragment slice (8 E4M3 codes).
__device__ __forceinline__ f16x8 decode8(uint32_t lo, uint32_t hi, uint32_t sw) {
  const float sc = __uint_as_float(sw);
  const _Float16 m = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sw & 0xFFFFu));
  const f16x2 m2 = {m, m};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, sc, false) * m2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, sc, true) * m2;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, sc, false) * m2;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, sc, true) * m2;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// Half of decode8: values 0..3 from lo (h = 0) or 4..7 from hi (h = 1), for
// placing between MFMAs.
__device__ __forceinline__ void decode8_half(f16x8& f, uint32_t w, uint32_t sw, int h) {
  const float sc = __uint_as_float(sw);
  // the mantissa factor in both halves: a splat of the low half, which the
  // packed multiply takes through its operand select (no extra instruction)
  const f16x2 sw2 = __builtin_bit_cast(f16x2, sw);
  const f16x2 m2 = {sw2[0], sw2[0]};
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, sc, false) * m2;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, sc, true) * m2;
  f[4 * h] = a[0]; f[4 * h + 1] = a[1]; f[4 * h + 2] = b[0]; f[4 * h + 3] = b[1];
}

template <int OP>
__global__ __launch_bounds__(256) void k_conv8w(const ConvParams p) {
  constexpr int MT = 256, NT = 256, WM = 2, KB = 4;
  constexpr int WTM = 128, WTN = 128, RM = 4, RN = 4;
  constexpr bool A_ROWS = (OP != OP_DGRAD);
  constexpr bool B_ROWS = (OP == OP_WGRAD);
  constexpr int PL = 304;                      // line-block pitch
  constexpr int PK = 272;                      // k-row pitch
  constexpr int GK = 8 * PK + 16;              // 8 k rows (one k-block) + pad
  constexpr int SZL = 32 * PL, SZK = 4 * GK;
  constexpr int A_SZ = A_ROWS ? SZL : SZK, B_SZ = B_ROWS ? SZL : SZK;
  constexpr int SCL = 32 * 16;
  constexpr int A_C = 0, B_C = A_SZ, A_S = A_SZ + B_SZ, B_S = A_S + SCL;
  constexpr int STAGE = A_S + 2 * SCL;
  constexpr int NST = 4;
  constexpr int LUT = NST * STAGE;
  static_assert(STAGE % 16 == 0, "16-byte aligned stages");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * STAGE + 1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx<OP, MT, NT, KB> t;
  if (!t.init(p, tid)) return;
  const bool is_a = t.is_a;  // uniform per wave: the first two waves stage A

  *reinterpret_cast<uint32_t*>(lds + LUT + tid * 4) = scale_word8(static_cast<uint32_t>(tid), kShift);

  // this thread's staging addresses (every thread stages one block a step):
  // line layout, row r of the block is line r of line block lblk at the
  // k-block's slot; k-row layout, row r is k row 8 slot + r at column 8 lblk
  const int slot = ((t.kbl & 1) << 1) | ((t.kbl >> 1) & 1);
  const bool rows = is_a ? A_ROWS : B_ROWS;
  const int st_code = (is_a ? A_C : B_C) + (rows ? t.lblk * PL + slot * 8 : slot * GK + t.lblk * 8);
  const int st_row = rows ? 32 : PK;
  const int st_scale = (is_a ? A_S : B_S) + t.lblk * 16 + slot * 4;

  const uint8_t* my_codes = is_a ? p.a_codes : p.b_codes;
  const uint8_t* my_scales = is_a ? p.a_scales : p.b_scales;
  KWalk<OP, MT, NT, KB> walk;
  walk.init(p, t);
  uint32_t s_fetch = 0;  // k offset (s * KB) of the next fetch
  auto fetch = [&](RawBlock<FMT_E4M3>& g) {
    uint32_t blk;
    const bool ok = walk.next(s_fetch, blk);
    g.load(my_codes, my_scales, blk, ok);
    s_fetch += KB;
  };
  uint32_t sws;  // scale word of the block being staged
  auto lookup_scale = [&](const RawBlock<FMT_E4M3>& g) {
    sws = *reinterpret_cast<const uint32_t*>(lds + LUT + ((g.scale & g.mask) << 2));
  };
  // rows r0, r0+1 of the staged block into stage `base`.  A padding block
  // carries the codes of block 0 with a zero scale word: its codes are
  // finite (a quantized tensor holds no NaN code), so it decodes to zeros.
  auto write_rows = [&](const RawBlock<FMT_E4M3>& g, uint8_t* base, int r0) {
#pragma unroll
    for (int r = r0; r < r0 + 2; ++r)
      *reinterpret_cast<u32x2v*>(base + st_code + r * st_row) = u32x2v{g.w[2 * r], g.w[2 * r + 1]};
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragment read addresses: fragment i adds 4 pitches (line layout) or 32
  // columns (k rows); the scale words of fragment i are 64 bytes further
  const int l32 = lane & 31, half = lane >> 5;
  const int line_off = (l32 >> 3) * PL + (l32 & 7) * 32 + half * 16;
  const int krow_off = half * 2 * GK + ((lane & 15) >> 1) * PK + ((lane >> 4) & 1) * 16 + (lane & 1) * 8;
  const int a_code = A_C + (A_ROWS ? wm * 16 * PL + line_off : krow_off + wm * 128);
  const int b_code = B_C + (B_ROWS ? wn * 16 * PL + line_off : krow_off + wn * 128);
  const int a_scale = A_S + (wm * 16 + (l32 >> 3)) * 16 + half * 8;
  const int b_scale = B_S + (wn * 16 + (l32 >> 3)) * 16 + half * 8;
  // raw fragments of two stages: .xy slice 0, .zw slice 1; scale words .x, .y
  u32x4v ra[2][RM], rb[2][RN];
  u32x2v sa[2][RM], sbv[2][RN];
  auto read_code = [&](const uint8_t* q, bool line) -> u32x4v {
    if (line) return *reinterpret_cast<const u32x4v*>(q);
    const auto s0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2v*)(q));
    const auto s1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2v*)(q + GK));
    return u32x4v{static_cast<uint32_t>(s0[0]), static_cast<uint32_t>(s0[1]), static_cast<uint32_t>(s1[0]),
                  static_cast<uint32_t>(s1[1])};
  };
  // part q (0..3) of the raw fragments of a stage: A and B fragment q with
  // their scale words
  auto read_raw = [&](auto set_c, const uint8_t* base, int q) {
    constexpr int Q = decltype(set_c)::value;
    ra[Q][q] = read_code(base + a_code + q * (A_ROWS ? 4 * PL : 32), A_ROWS);
    sa[Q][q] = *reinterpret_cast<const u32x2v*>(base + a_scale + q * 64);
    rb[Q][q] = read_code(base + b_code + q * (B_ROWS ? 4 * PL : 32), B_ROWS);
    sbv[Q][q] = *reinterpret_cast<const u32x2v*>(base + b_scale + q * 64);
  };
  auto dec = [&](const u32x4v& r, const u32x2v& s, int slice) -> f16x8 {
    return slice ? decode8(r.z, r.w, s.y) : decode8(r.x, r.y, s.x);
  };
  // half h of the slice-`slice` fragment of raw r into f
  auto dech = [&](f16x8& f, const u32x4v& r, const u32x2v& s, int slice, int h) {
    if (slice) decode8_half(f, h ? r.w : r.z, s.y, h);
    else decode8_half(f, h ? r.y : r.x, s.x, h);
  };
  f16x8 fa0[RM], fa1[RM];  // A fragments of slice 0 and slice 1

  // One column j of a slice: MFMA i is followed by work unit i (a few VALU
  // operations and LDS accesses), each closed by a scheduling barrier.
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
  // slice-0 column-0 B fragment fbc decoded): slice 0 decodes the slice-1 A
  // fragments and the next B fragment; slice 1 the next B fragment and the
  // next step's slice-0 A fragments (set Q, read from stage (s+1)%4 during
  // slice-0 column 0).  The block in G is staged into stage wr_c and G
  // refilled two steps ahead; a barrier at the end where bar_c is set.  Stage
  // offsets are compile-time constants.
  f16x8 fbc;
  auto step = [&](auto set_c, RawBlock<FMT_E4M3>& G, auto nxt_c, auto wr_c, auto bar_c) {
    constexpr int P = decltype(set_c)::value, Q = P ^ 1;
    uint8_t* wbase = lds + decltype(wr_c)::value;
    const uint8_t* nbase = lds + decltype(nxt_c)::value;
    f16x8 fbA, fbB;
    // slice 0
    column(fa0, fbc, 0,
           [&] { read_raw(IC<Q>{}, nbase, 0); dech(fa1[0], ra[P][0], sa[P][0], 1, 0); },
           [&] { read_raw(IC<Q>{}, nbase, 1); dech(fa1[0], ra[P][0], sa[P][0], 1, 1); },
           [&] { read_raw(IC<Q>{}, nbase, 2); dech(fbA, rb[P][1], sbv[P][1], 0, 0); },
           [&] { read_raw(IC<Q>{}, nbase, 3); dech(fbA, rb[P][1], sbv[P][1], 0, 1); });
    column(fa0, fbA, 1,
           [&] { lookup_scale(G); dech(fa1[1], ra[P][1], sa[P][1], 1, 0); },
           [&] { write_rows(G, wbase, 0); dech(fa1[1], ra[P][1], sa[P][1], 1, 1); },
           [&] { write_rows(G, wbase, 2); dech(fbB, rb[P][2], sbv[P][2], 0, 0); },
           [&] { write_rows(G, wbase, 4); dech(fbB, rb[P][2], sbv[P][2], 0, 1); });
    column(fa0, fbB, 2,
           [&] { write_rows(G, wbase, 6); dech(fa1[2], ra[P][2], sa[P][2], 1, 0); },
           [&] { fetch(G); dech(fa1[2], ra[P][2], sa[P][2], 1, 1); },
           [&] { *reinterpret_cast<uint32_t*>(wbase + st_scale) = sws; dech(fbA, rb[P][3], sbv[P][3], 0, 0); },
           [&] { dech(fbA, rb[P][3], sbv[P][3], 0, 1); });
    column(fa0, fbA, 3,
           [&] { dech(fa1[3], ra[P][3], sa[P][3], 1, 0); },
           [&] { dech(fa1[3], ra[P][3], sa[P][3], 1, 1); },
           [&] { dech(fbB, rb[P][0], sbv[P][0], 1, 0); },
           [&] { dech(fbB, rb[P][0], sbv[P][0], 1, 1); });
    // slice 1 (fa0 is free: it takes the next step's slice-0 A fragments)
    column(fa1, fbB, 0,
           [&] { dech(fbA, rb[P][1], sbv[P][1], 1, 0); },
           [&] { dech(fbA, rb[P][1], sbv[P][1], 1, 1); },
           [&] { dech(fa0[0], ra[Q][0], sa[Q][0], 0, 0); },
           [&] { dech(fa0[0], ra[Q][0], sa[Q][0], 0, 1); });
    column(fa1, fbA, 1,
           [&] { dech(fbB, rb[P][2], sbv[P][2], 1, 0); },
           [&] { dech(fbB, rb[P][2], sbv[P][2], 1, 1); },
           [&] { dech(fa0[1], ra[Q][1], sa[Q][1], 0, 0); },
           [&] { dech(fa0[1], ra[Q][1], sa[Q][1], 0, 1); });
    column(fa1, fbB, 2,
           [&] { dech(fbA, rb[P][3], sbv[P][3], 1, 0); },
           [&] { dech(fbA, rb[P][3], sbv[P][3], 1, 1); },
           [&] { dech(fa0[2], ra[Q][2], sa[Q][2], 0, 0); },
           [&] { dech(fa0[2], ra[Q][2], sa[Q][2], 0, 1); });
    column(fa1, fbA, 3,
           [&] { dech(fa0[3], ra[Q][3], sa[Q][3], 0, 0); },
           [&] { dech(fa0[3], ra[Q][3], sa[Q][3], 0, 1); },
           [&] { dech(fbc, rb[Q][0], sbv[Q][0], 0, 0); },
           [&] {
             dech(fbc, rb[Q][0], sbv[Q][0], 0, 1);
             if constexpr (decltype(bar_c)::value) __syncthreads();
           });
  };

  const int nsteps = (t.kb_end - t.kb_begin + KB - 1) / KB;
  if (nsteps > 0) {
    RawBlock<FMT_E4M3> g0, g1;  // the blocks that even and odd steps stage
    auto stage_block = [&](const RawBlock<FMT_E4M3>& g, uint8_t* base) {
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
    for (int i = 0; i < RM; ++i) fa0[i] = dec(ra[0][i], sa[0][i], 0);
    fbc = dec(rb[0][0], sbv[0][0], 0);
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
  // the fp16 fragments held g * B * 2^-2: one accumulator unit is 2^-4
  store_tile<OP, MT, NT, KB, WTM, WTN, RM, RN>(p, t, acc, lane, wm, wn, pow2(2 * kShift));
}

}  // namespace

namespace gemm {

// The 256x256 E4M3 decode-at-read kernel; false (nothing launched) where its
// K walk needs the division-based block search (an innermost K extent below
// 4 k-blocks).
bool launch_conv8(int op, const ConvParams& p, dim3 grid, hipStream_t s) {
  if (!kwalk_ok(op, p, 4)) return false;
  switch (op) {
    case OP_FWD: hipLaunchKernelGGL((k_conv8w<OP_FWD>), grid, dim3(256), 0, s, p); break;
    case OP_DGRAD: hipLaunchKernelGGL((k_conv8w<OP_DGRAD>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((k_conv8w<OP_WGRAD>), grid, dim3(256), 0, s, p); break;
  }
  return true;
}

}  // namespace gemm
}  // namespace mx
