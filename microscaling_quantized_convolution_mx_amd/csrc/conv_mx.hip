// Convolution GEMMs on the original microscaling format (E8M0 scale per
// 32x32 square block, E2M1 elements, no tensor scale) with gfx950's scaled
// FP4 MFMA (MicroQonv, arXiv 2609.28358, §II-D, §IV-B).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 takes, per lane, 32 consecutive K values
// of one row (A) or column (B) and one E8M0 scale for them: lane l holds
// row / column l%32 and K half l/32.  A 32x32 square block is therefore
// exactly one half-wave operand with one scale, whichever of its two
// directions K runs along, so every operand is read straight from the
// quantized blocks: no decode, no im2col, and the same blocks serve the
// forward, data-gradient and weight-gradient GEMMs.
//
// Blocks are stored as 32 rows of 16 bytes (channel rows for activations
// and gradients, output-channel rows for weights).  Where K runs along a
// block's rows (wgrad's A and B, fwd's A) a lane reads its 16 bytes
// directly; where K runs down the columns (fwd's B, dgrad's A and B) two
// transposing LDS reads (ds_read_b64_tr_b4: 16x16 nibble transpose within
// each group of 16 lanes) gather the 32 nibbles of a column.
//
// Tile 256x256, 4 waves of 128x128 (4x4 MFMAs of 32x32).  One K step is
// 128 K values: 4 32-blocks per row / column block of the tile, two MFMA
// k-slices of 16 MFMAs per wave behind one barrier.  Every thread copies
// eight 16-byte block rows per step from global memory into one of three
// LDS stages (the blocks unchanged).  The rows are fetched into registers
// two steps before they are written to LDS, so an L2 or HBM load has two
// steps of MFMAs to arrive.  Tile placement, the stride phases of dgrad and
// the epilogue are those of the generic kernel.
#include "conv_kernels.h"

namespace mx {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2v;

constexpr int kKB = kMxStepBlocks;  // 32-blocks along K per step
constexpr int kMxB = 512;           // bytes of one 32x32 E2M1 block

template <int I>
struct Idx {
  static constexpr int value = I;
};
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f(Idx<I>{}), ...); }(std::make_integer_sequence<int, N>());
}

// TILE x TILE outputs per workgroup, 4 waves of TILE/2 x TILE/2.
template <int OP, int TILE>
__global__ __launch_bounds__(256) void k_conv_mx(const ConvParams p) {
  constexpr int MT = TILE, NT = TILE, WM = 2;
  constexpr int WTM = TILE / 2, WTN = TILE / 2, RM = TILE / 64, RN = TILE / 64;
  constexpr int NLB = TILE / 32;                     // line blocks (32 lines) of an operand in the tile
  constexpr int NQ = NLB / 2;                        // block rows a thread stages per operand and step
  constexpr int kOpnd = NLB * kKB * kMxB;            // one operand of a stage: NLB line blocks x kKB k-blocks
  constexpr int kStage = 2 * kOpnd + 2 * NLB * kKB;  // codes of A and B, then scales [A: kKB x NLB][B: kKB x NLB]
  static_assert(RM == NQ && RN == NQ, "one staged row of each operand per MFMA row of a k-slice");
  // K runs along the stored rows of A for fwd and wgrad, of B for wgrad
  constexpr bool A_DIRECT = (OP != OP_DGRAD);
  constexpr bool B_DIRECT = (OP == OP_WGRAD);
  __shared__ __attribute__((aligned(16))) uint8_t lds[3 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx<OP, MT, NT, 4> t;  // placement, dgrad phase and epilogue geometry (8-column units)
  if (!t.init(p, tid)) return;

  // 32-block counts
  const int cbi = p.c_in >> 5, cbo = p.c_out >> 5, nbk = p.n >> 5;
  const int rb0 = (t.rb0 * 8) >> 5;               // first row block of the tile
  const int cb0 = (t.cb0 * 8) >> 5;               // first column block
  const int nrb = p.M >> 5;                       // row blocks of the GEMM
  const int ncb = (t.ncb_launch * 8) >> 5;        // column blocks of the launch
  // K extent in 32-blocks and this launch's range of K steps (kKB blocks each)
  int k_total;
  if constexpr (OP == OP_FWD) k_total = p.k_h * p.k_w * cbi;
  else if constexpr (OP == OP_DGRAD) k_total = t.nkh * t.nkw * cbo;
  else k_total = p.ho * p.wo * nbk;
  const int nsteps_all = (k_total + kKB - 1) / kKB;
  int s_begin = 0, s_end = nsteps_all;
  if constexpr (OP == OP_WGRAD) {
    s_begin = t.bz * p.ks_split;
    s_end = min(nsteps_all, s_begin + p.ks_split);
    if (s_begin > s_end) s_begin = s_end;
  }
  // k-blocks past this launch's range read as zeros
  const int k_end = min(k_total, kKB * s_end);

  // Staging: thread t copies row (t & 31) of the blocks (operand, line block
  // lb, k-block kb) with kb = (t >> 5) & 3 and lb = (t >> 7) + 2j,
  // j = 0..NQ-1, for A (q = j) and for B (q = NQ + j).
  const int row = tid & 31, kb = (tid >> 5) & 3, lbq = tid >> 7;
  auto q_lb = [&](int q) { return lbq + 2 * (q % NQ); };
  int gline[2 * NQ];
  bool gline_ok[2 * NQ];
  // column-block geometry of B (fixed over the K loop)
  int col_y[NQ], col_x[NQ], col_nb[NQ], col_cib[NQ];
#pragma unroll
  for (int q = 0; q < 2 * NQ; ++q) {
    const int lb = q_lb(q);
    if (q < NQ) {
      gline[q] = rb0 + lb;
      gline_ok[q] = gline[q] < nrb;
    } else {
      const int cb = cb0 + lb;
      gline[q] = cb;
      gline_ok[q] = cb < ncb;
      const int i = q - NQ;
      col_y[i] = col_x[i] = col_nb[i] = col_cib[i] = 0;
      if constexpr (OP == OP_FWD) {
        const int pos = cb / nbk;
        col_nb[i] = cb - pos * nbk;
        const int ho = pos / p.wo;
        col_y[i] = ho * p.sh - p.ph;
        col_x[i] = (pos - ho * p.wo) * p.sw - p.pw;
      } else if constexpr (OP == OP_DGRAD) {
        const int pos = cb / nbk;
        col_nb[i] = cb - pos * nbk;
        const int hq = pos / t.wp;
        const int h = t.phh + p.sh * hq, w = t.phw + p.sw * (pos - hq * t.wp);
        // dY row of tap kh = kh0 + sh*a is (h + ph - kh0)/sh - a (exact)
        col_y[i] = (h + p.ph - t.kh0) / p.sh;
        col_x[i] = (w + p.pw - t.kw0) / p.sw;
      } else {
        const int tap = cb / cbi;
        col_cib[i] = cb - tap * cbi;
        const int kh = tap / p.k_w;
        col_y[i] = kh - p.ph;
        col_x[i] = (tap - kh * p.k_w) - p.pw;
      }
    }
  }
  FastDiv div_in, div_b;
  if constexpr (OP == OP_FWD) { div_in.init(cbi); div_b.init(p.k_w); }
  else if constexpr (OP == OP_DGRAD) { div_in.init(cbo); div_b.init(t.nkw > 0 ? t.nkw : 1); }
  else { div_in.init(nbk); div_b.init(p.wo); }

  // global block index of block row q at k-block k (and whether it exists)
  auto locate = [&](int q, int k, uint32_t& blk) -> bool {
    const uint32_t outer = div_in.div(static_cast<uint32_t>(k));
    const uint32_t inner = static_cast<uint32_t>(k) - outer * div_in.d;
    const uint32_t a = div_b.div(outer);
    const uint32_t b = outer - a * div_b.d;
    const bool kin = k < k_end;
    if (q < NQ) {
      const uint32_t rb = static_cast<uint32_t>(gline[q]);
      if constexpr (OP == OP_FWD) blk = ((a * p.k_w + b) * cbo + rb) * cbi + inner;                 // W[tap][co][ci]
      else if constexpr (OP == OP_DGRAD)
        blk = (((t.kh0 + p.sh * a) * p.k_w + (t.kw0 + p.sw * b)) * cbo + inner) * cbi + rb;         // W[tap][co][ci]
      else blk = ((a * p.wo + b) * cbo + rb) * nbk + inner;                                            // dY[pos][co][n]
      return gline_ok[q] && kin;
    }
    const int i = q - NQ;
    int y, x;
    bool inb;
    if constexpr (OP == OP_FWD) {
      y = col_y[i] + static_cast<int>(a);
      x = col_x[i] + static_cast<int>(b);
      inb = static_cast<uint32_t>(y) < static_cast<uint32_t>(p.h) && static_cast<uint32_t>(x) < static_cast<uint32_t>(p.w);
      blk = ((static_cast<uint32_t>(y) * p.w + x) * cbi + inner) * nbk + col_nb[i];                // X[pos][ci][n]
    } else if constexpr (OP == OP_DGRAD) {
      y = col_y[i] - static_cast<int>(a);
      x = col_x[i] - static_cast<int>(b);
      inb = static_cast<uint32_t>(y) < static_cast<uint32_t>(p.ho) && static_cast<uint32_t>(x) < static_cast<uint32_t>(p.wo);
      blk = ((static_cast<uint32_t>(y) * p.wo + x) * cbo + inner) * nbk + col_nb[i];               // dY[pos][co][n]
    } else {
      y = col_y[i] + static_cast<int>(a) * p.sh;
      x = col_x[i] + static_cast<int>(b) * p.sw;
      inb = static_cast<uint32_t>(y) < static_cast<uint32_t>(p.h) && static_cast<uint32_t>(x) < static_cast<uint32_t>(p.w);
      blk = ((static_cast<uint32_t>(y) * p.w + x) * cbi + col_cib[i]) * nbk + inner;               // X[pos][ci][n]
    }
    return gline_ok[q] && kin && inb;
  };

  // one step's block rows in registers: codes, scale (used by row 0) and
  // whether the block exists.  The mask is applied when the rows are
  // written to LDS, so that nothing waits for a load before then.
  struct Raw {
    uint4 v[2 * NQ];
    uint32_t sc[2 * NQ];
    uint32_t mask[2 * NQ];
  };
  Raw r0, r1;
  auto fetch_one = [&](Raw& raw, int step, int q) {
    const int k = kKB * step + kb;
    uint32_t blk = 0;
    const bool ok = locate(q, k, blk);
    const uint8_t* codes = q < NQ ? p.a_codes : p.b_codes;
    const uint8_t* scales = q < NQ ? p.a_scales : p.b_scales;
    const uint64_t b = ok ? blk : 0u;
    raw.v[q] = *reinterpret_cast<const uint4*>(codes + b * kMxB + row * 16);
    raw.sc[q] = scales[b];
    raw.mask[q] = ok ? ~0u : 0u;
  };
  auto fetch = [&](Raw& raw, int step) {
#pragma unroll
    for (int q = 0; q < 2 * NQ; ++q) fetch_one(raw, step, q);
  };
  // stage layout: block (lb, kb) of an operand at (lb * kKB + kb) * kMxB;
  // scales [kb][lb] (A at 2*kOpnd, B NLB*kKB bytes later)
  auto stage_write = [&](const Raw& raw, uint8_t* st) {
#pragma unroll
    for (int q = 0; q < 2 * NQ; ++q) {
      const int lb = q_lb(q);
      const uint32_t m = raw.mask[q];
      // a block outside the operand is zeros with scale 2^0
      *reinterpret_cast<uint4*>(st + (q < NQ ? 0 : kOpnd) + (lb * kKB + kb) * kMxB + row * 16) =
          make_uint4(raw.v[q].x & m, raw.v[q].y & m, raw.v[q].z & m, raw.v[q].w & m);
      if (row == 0)
        st[2 * kOpnd + (q < NQ ? 0 : NLB * kKB) + kb * NLB + lb] = static_cast<uint8_t>((raw.sc[q] & m) | (127u & ~m));
    }
  };

  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int l32 = lane & 31, half = lane >> 5;
  // operand of line block lb, k-slice j, for this lane: block (lb, 2j +
  // half); direct = its row l32; transposed = its column l32, gathered 16
  // rows at a time (lane group g = lane/16 covers columns 16*(g%2) .. +15)
  const int direct_off = half * kMxB + l32 * 16;
  const int trans_off = half * kMxB + (lane & 15) * 16 + ((lane >> 4) & 1) * 8;
  auto read_opnd = [&](const uint8_t* base, int lb, int j, bool direct) -> i32x8 {
    const uint8_t* blk = base + (lb * kKB + 2 * j) * kMxB;
    if (direct) {
      const uint4 v = *reinterpret_cast<const uint4*>(blk + direct_off);
      return i32x8{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w), 0, 0, 0, 0};
    }
    const i32x2v r0 = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2v*)(blk + trans_off));
    const i32x2v r1 = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2v*)(blk + trans_off + 16 * 16));
    return i32x8{r0.x, r0.y, r1.x, r1.y, 0, 0, 0, 0};
  };
  // the MFMA operands of one k-slice: fragments and scale words (byte i of
  // a scale word is the scale of fragment i: the MFMA's op_sel)
  struct Frags {
    i32x8 a[RM], b[RN];
    int sa, sb;
  };
  Frags fA, fB;
  auto scale_word = [&](const uint8_t* q) -> int {
    if constexpr (RM == 4) return *reinterpret_cast<const int*>(q);
    else return static_cast<int>(*reinterpret_cast<const uint16_t*>(q));
  };
  auto read_frags = [&](const uint8_t* st, int j, Frags& f) {
    // the wave's line blocks of k-block 2j + half
    f.sa = scale_word(st + 2 * kOpnd + (2 * j + half) * NLB + wm * RM);
    f.sb = scale_word(st + 2 * kOpnd + NLB * kKB + (2 * j + half) * NLB + wn * RN);
#pragma unroll
    for (int i = 0; i < RM; ++i) f.a[i] = read_opnd(st, wm * RM + i, j, A_DIRECT);
#pragma unroll
    for (int i = 0; i < RN; ++i) f.b[i] = read_opnd(st + kOpnd, wn * RN + i, j, B_DIRECT);
  };

  // Step s, on stage s%3, with slice 0's operands read into fA during step
  // s-1:
  //   write the rows of step s+2 (fetched two steps earlier) into stage
  //   (s+2)%3, last read during step s-1;
  //   read slice 1 into fB; the MFMAs on fA, with fetches of step s+4 for A;
  //   read slice 0 of step s+1 from stage (s+1)%3 (complete since the
  //   barrier of step s-1) into fA; the MFMAs on fB, with fetches for B;
  //   barrier.
  // Steps run in pairs so that the two row register sets alternate
  // statically, with no exit in between (an exit there makes the compiler
  // spill the accumulators); fetches at or past the last step give zero
  // rows, so the extra step of an odd count adds nothing.
  const int nsteps = s_end - s_begin;
  auto slice = [&](const Frags& F, Raw& raw, int fs, int q0) {
    static_for<RM>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      static_for<RN>([&](auto jc) {
        constexpr int J = decltype(jc)::value;
        acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[I], F.b[J], acc[I][J], 4, 4, I, F.sa, J, F.sb);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (J == 0) {
          fetch_one(raw, fs, q0 + I);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    });
  };
  auto step = [&](int s, const uint8_t* cur, const uint8_t* next_st, uint8_t* write_st, Raw& raw) {
    const int fs = s_begin + s + 4;
    stage_write(raw, write_st);
    read_frags(cur, 1, fB);
    __builtin_amdgcn_sched_barrier(0);
    slice(fA, raw, fs, 0);
    read_frags(next_st, 0, fA);
    __builtin_amdgcn_sched_barrier(0);
    slice(fB, raw, fs, NQ);
    // The MFMAs carry no ordering of their own: without a use here, the
    // first step of a pair has its MFMAs emitted after the barrier below,
    // leaving the MFMA pipe idle while the waves wait there.  An empty asm
    // that takes each accumulator keeps them ahead of the barrier.
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) asm volatile("" : "+a"(acc[i][j]));
    __syncthreads();
  };
  if (nsteps > 0) {
    fetch(r0, s_begin);
    fetch(r1, s_begin + 1);
    stage_write(r0, lds);
    stage_write(r1, lds + kStage);
    fetch(r0, s_begin + 2);
    fetch(r1, s_begin + 3);
    __syncthreads();
    read_frags(lds, 0, fA);
    int c = 0;  // stage of step s
    for (int s = 0; s < nsteps; s += 2) {
      const int c1 = c == 2 ? 0 : c + 1, c2 = c1 == 2 ? 0 : c1 + 1;
      // step s writes rows s+2 (r0) into c2; step s+1 writes rows s+3 (r1) into c
      step(s, lds + c * kStage, lds + c1 * kStage, lds + c2 * kStage, r0);
      step(s + 1, lds + c1 * kStage, lds + c2 * kStage, lds + c * kStage, r1);
      c = c2;
    }
  }

  store_tile<OP, MT, NT, 4, WTM, WTN, RM, RN>(p, t, acc, lane, wm, wn);
}

}  // namespace

namespace gemm {

void launch_mx(int op, int tile, const ConvParams& p, dim3 grid, hipStream_t s) {
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, p); };
  if (tile == 128) {
    switch (op) {
      case OP_FWD: go(k_conv_mx<OP_FWD, 128>); break;
      case OP_DGRAD: go(k_conv_mx<OP_DGRAD, 128>); break;
      default: go(k_conv_mx<OP_WGRAD, 128>); break;
    }
  } else {
    switch (op) {
      case OP_FWD: go(k_conv_mx<OP_FWD, 256>); break;
      case OP_DGRAD: go(k_conv_mx<OP_DGRAD, 256>); break;
      default: go(k_conv_mx<OP_WGRAD, 256>); break;
    }
  }
}

}  // namespace gemm
}  // namespace mx
