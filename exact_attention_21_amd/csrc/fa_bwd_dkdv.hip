// dK/dV pass instantiations for d = 64 and for non-causal d = 128, and the
// dispatcher of the pass (causal d = 128 comes from fa_bwd_dkdv_ilp.hip).
#include "fa_bwd_dkdv.h"

namespace fa {

hipError_t launch_bwd_dkdv(const BwdParams &p, int dtype, int d, int causal, int grid,
                           hipStream_t st) {
  if (d == 128 && causal) return launch_bwd_dkdv_causal128(p, dtype, grid, st);
  if (dtype == 1)
    return d == 128 ? launch_dkdv_c<BF16, 128, false>(p, grid, st)
                    : (causal ? launch_dkdv_c<BF16, 64, true>(p, grid, st) : launch_dkdv_c<BF16, 64, false>(p, grid, st));
  return d == 128 ? launch_dkdv_c<F16, 128, false>(p, grid, st)
                  : (causal ? launch_dkdv_c<F16, 64, true>(p, grid, st) : launch_dkdv_c<F16, 64, false>(p, grid, st));
}

}  // namespace fa
