// Kernel parameter blocks and launchers shared between the kernel sources and
// the C-ABI layer.  Host-and-device header; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Keys per K/V tile of the forward kernel, by head dim.
constexpr int FWD_BN_D128 = 64;
constexpr int FWD_BN_D64 = 64;

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

hipError_t launch_bwd(const BwdParams &p, int dtype, int d, int causal, int grid, long rows,
                      hipStream_t st);

hipError_t launch_fwd(const FwdParams &p, int dtype, int d, int causal, int qb, int grid,
                      hipStream_t st);

}  // namespace fa
