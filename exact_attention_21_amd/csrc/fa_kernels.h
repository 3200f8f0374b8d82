// Kernel parameter blocks and launchers shared between the kernel sources and
// the C-ABI layer.  Host-and-device header; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Keys per K/V tile (one pipeline step) of the forward kernel.
constexpr int FWD_BN = 32;
// Query blocks of 32 rows per wave for head dim 128, and whether the output
// accumulator is kept in AGPRs (set together with the compiler's MFMA register
// form for fa_fwd.hip).
#ifndef FWD_QB_D128
#define FWD_QB_D128 1
#endif
#ifndef FWD_O_IN_AGPR
#define FWD_O_IN_AGPR (FWD_QB_D128 == 2)
#endif
// Waves per SIMD the forward kernel is compiled for (occupancy target).
#ifndef FWD_WAVES_PER_SIMD
#define FWD_WAVES_PER_SIMD 3
#endif

struct FwdParams {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int N;            // sequence length
  int n_qtiles;     // ceil(N / BM)
  int xcd_grouped;  // 1: B*H is a multiple of 8 and heads are grouped per XCD
  float scale_log2; // scale * log2(e)
};

// Backward tiling: keys per workgroup and query rows per inner step.
constexpr int BWD_BN = 128;
constexpr int BWD_BM = 64;

struct BwdParams {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *dq_acc;    // fp32 [B][H][N][d] workspace
  float *dws;       // fp32 [B][H][N] workspace: D = rowsum(dO * O)
  int N;
  int n_ktiles;     // ceil(N / BWD_BN)
  int xcd_grouped;
  float scale;
  float scale_log2;
};

// D = rowsum(dO * O) and zeroed dQ accumulator (reads p.o, p.dout; writes p.dws, p.dq_acc)
hipError_t launch_bwd_pre(const BwdParams &p, int dtype, int d, long rows, hipStream_t st);
// main backward kernel (writes p.dk, p.dv, accumulates p.dq_acc)
hipError_t launch_bwd_main(const BwdParams &p, int dtype, int d, int causal, int grid,
                           hipStream_t st);
// dQ = scale * accumulator -> 16 bits (reads p.dq_acc, writes p.dq)
hipError_t launch_bwd_dq(const BwdParams &p, int dtype, long elems, hipStream_t st);

hipError_t launch_fwd(const FwdParams &p, int dtype, int d, int causal, int qb, int grid,
                      hipStream_t st);

}  // namespace fa
