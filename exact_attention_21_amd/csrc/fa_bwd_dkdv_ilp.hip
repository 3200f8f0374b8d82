// The causal d = 128 dK/dV kernels, compiled with LLVM's iterative ILP
// instruction scheduler (-amdgpu-sched-strategy=iterative-ilp, set for this
// file in build.py).  Interleaved timings on one MI355X: the pass at B=4 H=32
// N=8192 causal ran 1.9-2.4 % faster and at N=16384 1.1 % faster than with
// the default scheduler; for the other dK/dV variants (d = 64, non-causal) it
// was 1 % slower, and the dQ pass spills under it, so only these use it.
#include "fa_bwd_dkdv.h"

namespace fa {

hipError_t launch_bwd_dkdv_causal128(const BwdParams &p, int dtype, int grid, hipStream_t st) {
  return dtype == 1 ? launch_dkdv_c<BF16, 128, true>(p, grid, st) : launch_dkdv_c<F16, 128, true>(p, grid, st);
}

}  // namespace fa
