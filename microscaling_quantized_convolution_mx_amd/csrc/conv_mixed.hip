// Instantiations of the generic convolution GEMM for the operand formats
// beyond the three uniform hot-path ones, compiled apart from conv.hip:
//   - E3M2 in all three GEMMs (the FP6 with the wider range);
//   - MicroQonv+ (§IV-D, Table VI): E2M1 weights and output gradients with
//     FP6 activations, E3M2 or E2M3, in the forward (W x X') and
//     weight-gradient (dY x X'^T) GEMMs; the data gradient (W^T x dY) has no
//     activation operand and runs all-E2M1.
// Both FP6 formats and E2M1 decode exactly to fp16, so a mixed pair shares
// the fp16 MFMA.  On the 256x256 tile these pairs run on the kernel of FP6
// activations in conv_staged.hip.
#include "conv_kernels.h"

namespace mx {
namespace gemm {

bool launch_mixed(int op, const ConvParams& p, int fmt_a, int fmt_b, const Tile& t, dim3 grid, hipStream_t s) {
  // the 256x256 tile: FP6 activations on the kernel that decodes at staging
  if (t.mt == 256 && t.nt == 256 && launch_staged(op, fmt_a, fmt_b, p, grid, s)) return true;
  if (fmt_a == FMT_E3M2 && fmt_b == FMT_E3M2) {
    switch (op) {
      case OP_FWD: launch_generic<OP_FWD, FMT_E3M2, FMT_E3M2>(p, t, grid, s); return true;
      case OP_DGRAD: launch_generic<OP_DGRAD, FMT_E3M2, FMT_E3M2>(p, t, grid, s); return true;
      case OP_WGRAD: launch_generic<OP_WGRAD, FMT_E3M2, FMT_E3M2>(p, t, grid, s); return true;
      default: return false;
    }
  }
  if (fmt_a != FMT_E2M1 || (op != OP_FWD && op != OP_WGRAD)) return false;
  if (fmt_b == FMT_E3M2) {
    if (op == OP_FWD) launch_generic<OP_FWD, FMT_E2M1, FMT_E3M2>(p, t, grid, s);
    else launch_generic<OP_WGRAD, FMT_E2M1, FMT_E3M2>(p, t, grid, s);
    return true;
  }
  if (fmt_b == FMT_E2M3) {
    if (op == OP_FWD) launch_generic<OP_FWD, FMT_E2M1, FMT_E2M3>(p, t, grid, s);
    else launch_generic<OP_WGRAD, FMT_E2M1, FMT_E2M3>(p, t, grid, s);
    return true;
  }
  return false;
}

}  // namespace gemm
}  // namespace mx
