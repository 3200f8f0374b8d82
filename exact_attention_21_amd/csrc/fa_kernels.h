// Kernel parameter blocks and launchers shared between the kernel sources and
// the C-ABI layer.  Host-and-device header; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Keys per K/V tile (one pipeline step) of the forward kernel.
constexpr int FWD_BN = 32;
#ifndef FWD_NSLOT_D128
#define FWD_NSLOT_D128 3  // K/V ring slots of the d = 128 forward without dropout (tiles loaded NSLOT - 1 steps ahead)
#endif
#ifndef FWD_NSLOT_SPLIT
#define FWD_NSLOT_SPLIT 3  // the same for the split forward (decode shapes)
#endif
// Waves per SIMD the forward kernel is compiled for (occupancy target).
#ifndef FWD_WAVES_PER_SIMD
#define FWD_WAVES_PER_SIMD 3
#endif
// d = 64: query blocks per wave for N > 128, and the occupancy of the one-block
// kernel (one block at four waves per SIMD, 103-117 VGPRs: 1.3 % faster than two
// blocks at two)
#ifndef FWD_QB_D64
#define FWD_QB_D64 1
#endif
#ifndef FWD_WAVES_D64
#define FWD_WAVES_D64 4
#endif

// Sequence shape of a call.  Query-side tensors (Q, O, dO, dQ, LSE) have Nq
// rows per head, key-side ones (K, V, dK, dV) Nk.  Batch entry b has
// Lq = clamp(lq[b], 0, Nq) valid queries and Lk = clamp(lk[b], 0, Nk) valid
// keys; lq / lk NULL means all valid.  With the causal mask query i sees key j
// iff j <= i + Lk - Lq (the diagonal ends at the last query and the last key).
struct SeqShape {
  int Nq, Nk;
  int H;
  const int *lq, *lk;  // device int32 [B] or NULL
};

// Valid lengths of batch entry b (uniform across the workgroup: scalar loads).
__device__ __forceinline__ void seq_lengths(const SeqShape &s, int b, int &Lq, int &Lk) {
  Lq = s.lq ? min(max(s.lq[b], 0), s.Nq) : s.Nq;
  Lk = s.lk ? min(max(s.lk[b], 0), s.Nk) : s.Nk;
}

// Dropout on the attention weights: pair (i, j) of head bh is kept iff byte
// j % 4 of word i % 4 of Philox4x32-10(counter (j/4, i/4, bh, offset), key
// (k0, k1)) is >= p8; kept weights are scaled by `scale` = 256 / (256 - p8).
// p8 = 0: no dropout (the kernels without dropout are launched).
struct DropoutSpec {
  uint32_t p8, k0, k1, offset;
  float scale;
};

// Causal grids: heads per dispatch group (see grid_tile), chosen by the host.
// More heads per group end the grid on shorter tiles but keep more heads' K/V
// in use on an XCD at once (more L2 misses).  Four heads when every head has
// the same length and one head's K and V take at most 2 MiB (N d <= 2^19);
// pairs otherwise: with larger heads four of them raised the L2 misses by a
// third to a half for no measurable time, and with per-batch lengths the rank
// order inside a group is by tile index, which is by length only within one
// batch entry (a group of four spans two entries).
constexpr int CAUSAL_GROUP_SMALL = 4;
constexpr int CAUSAL_GROUP_PAIR = 2;
constexpr long CAUSAL_GROUP_SMALL_MAX_ND = 1L << 19;
// Heads of the final dispatch group of an XCD that holds `slots` workgroups
// at once: enough tiles for two rounds of its slots.
__host__ __device__ constexpr int causal_tail_heads(int ntiles, int slots) {
  return (2 * slots + ntiles - 1) / ntiles;
}

struct FwdParams {
  const void *q, *k, *v;
  void *o;
  float *lse;
  SeqShape seq;
  DropoutSpec drop;
  // split over key blocks: workgroup (head, query tile, split s) covers keys
  // [s * chunk, (s + 1) * chunk) and writes its normalised partial output and
  // LSE to opart [B*H][nsplit][Nq][d] / lpart [B*H][nsplit][Nq] (fp32)
  int nsplit, chunk;
  float *opart, *lpart;
  int n_qtiles;     // ceil(Nq / BM)
  int xcd_grouped;  // 1: B*H is a multiple of 8 and heads are grouped per XCD
  float scale_log2; // scale * log2(e)
  int causal_group; // causal: heads per dispatch group
};

// Backward tiling.  dQ pass: 128 query rows per workgroup, 32 keys per step.
// dK/dV pass: 128 keys per workgroup, 32 query rows per step.
constexpr int BWD_DQ_BM = 128;
constexpr int BWD_DKDV_BN = 128;
constexpr int BWD_DKDV_BM = 32;
#ifndef BWD_DQ_WAVES_PER_SIMD
#define BWD_DQ_WAVES_PER_SIMD 2
#endif
#ifndef BWD_DKDV_WAVES_PER_SIMD
#define BWD_DKDV_WAVES_PER_SIMD 2
#endif
// d = 64 fits more waves per SIMD
#ifndef BWD_DQ_WAVES_D64
#define BWD_DQ_WAVES_D64 4
#endif
#ifndef BWD_DKDV_WAVES_D64
#define BWD_DKDV_WAVES_D64 3
#endif
// Ring slots of the dK/dV pass: Q/dO tiles are loaded NSLOT - 1 steps ahead.
#ifndef BWD_DQ_NSLOT_D128
#define BWD_DQ_NSLOT_D128 3  // dQ pass K/V ring slots at d = 128 (loads run NSLOT - 1 steps ahead)
#endif
#ifndef BWD_DQ_KT_EARLY
#define BWD_DQ_KT_EARLY 4  // dQ pass (d = 128, no dropout): K^T column blocks read before the softmax
#endif
#ifndef BWD_DKDV_DROP_VF_LDS
#define BWD_DKDV_DROP_VF_LDS 3  // dK/dV pass with dropout, d = 128: V fragments kept in LDS
#endif
#ifndef BWD_DKDV_NSLOT
#define BWD_DKDV_NSLOT 2
#endif
constexpr int BWD_DKDV_STAT = 512;  // bytes of LSE2 and D per ring slot

struct BwdParams {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *dws;       // fp32 [B][H][Nq] workspace: -D = -rowsum(dO * O)
  float *lse2;      // fp32 [B][H][Nq] workspace: LSE * log2(e) (+inf for rows with LSE = -inf)
  SeqShape seq;
  DropoutSpec drop;
  int n_qtiles;     // ceil(Nq / BWD_DQ_BM)
  int n_ktiles;     // ceil(Nk / BWD_DKDV_BN)
  int xcd_grouped;
  float scale;
  float scale_log2;
  int causal_group;  // causal: heads per dispatch group
};

// -D = -rowsum(dO * O) and LSE * log2(e) (reads p.o, p.dout, p.lse; writes p.dws, p.lse2)
hipError_t launch_bwd_pre(const BwdParams &p, int dtype, int d, long rows, hipStream_t st);
// dQ pass (reads q, k, v, dout, dws, lse2; writes dq); grid = n_qtiles * B * H.
// pre != 0: it computes dws and lse2 itself (reads o and lse, writes dws, lse2)
hipError_t launch_bwd_dq(const BwdParams &p, int dtype, int d, int causal, int pre, int grid,
                         hipStream_t st);
// dK/dV pass (reads q, k, v, dout, dws, lse2; writes dk, dv); grid = n_ktiles * B * H
hipError_t launch_bwd_dkdv(const BwdParams &p, int dtype, int d, int causal, int grid,
                           hipStream_t st);

hipError_t launch_fwd(const FwdParams &p, int dtype, int d, int causal, int qb, int grid,
                      hipStream_t st);
// split-over-keys forward (grid = n_qtiles * nsplit * B * H), then the merge of
// the partials into o and lse (one wave per query row)
hipError_t launch_fwd_split(const FwdParams &p, int dtype, int d, int causal, int grid,
                            hipStream_t st);
hipError_t launch_fwd_combine(const FwdParams &p, int dtype, int d, long rows, hipStream_t st);
// decode forward (Nq = 1): one partial per wave, p.nsplit partials per head
// (a multiple of 4), p.chunk keys each (a multiple of fwd_decode_tile(d));
// grid = B * H * nsplit / 4; the partials are merged by launch_fwd_combine
constexpr int fwd_decode_tile(int d) { return d == 128 ? 32 : 64; }
hipError_t launch_fwd_decode(const FwdParams &p, int dtype, int d, int grid, hipStream_t st);

}  // namespace fa
