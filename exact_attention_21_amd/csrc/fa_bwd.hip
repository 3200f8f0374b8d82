// Attention backward for gfx950, with recomputation of the probabilities from
// the forward's log-sum-exp ("Flash Attention application", section
// "Recomputation": P is not stored, it is rebuilt in the backward; its v2
// section: the backward kernel's parallel schedule is what v2 reworked).
//
// The gradients are the calculus of O = softmax(scale Q K^T) V:
//   P = exp(scale S - LSE), dV = P^T dO, dP = dO V^T, D_i = rowsum(dO_i * O_i),
//   dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three kernels, none with atomics (so every output is bitwise reproducible):
//   bwd_pre_kernel   -D = -rowsum(dO * O) and LSE * log2(e), fp32 [B][H][Nq]
//   bwd_dq_kernel    one workgroup per 128 query rows, K/V tiles streamed through
//                    LDS (the forward's structure): S^T = K Q^T, dP^T = V dO^T,
//                    dS^T = P^T (dP^T - D), dQ^T += K^T dS^T; its PRE variant
//                    computes -D and LSE * log2(e) itself and stores them, so
//                    the full backward is two launches: dQ (PRE), then dK/dV
//   bwd_dkdv_kernel  one workgroup per 128 keys, Q/dO tiles streamed through LDS:
//                    S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS
// P and dS are recomputed in both passes (two extra tile products compared with
// a single pass that accumulates dQ with atomics), in exchange for no atomic
// traffic, no fp32 dQ accumulator and deterministic results.
//
// MFMA orientation follows the forward: in the query-major pass a lane owns one
// query and 16 keys of each 32x32 score block (the packed dS^T registers are
// directly the B operand of dQ^T += K^T dS^T, whose A operand is read from LDS
// with ds_read_b64_tr_b16); in the key-major pass a lane owns one key and 16
// queries (packed P and dS are the B operands of dV^T += dO^T P and
// dK^T += Q^T dS, with dO^T and Q^T read transposed from LDS).  Tiles reach LDS
// by direct buffer->LDS loads one step ahead, with XOR-swizzled rows (see the
// forward kernel).
//
// This file holds the row statistics and the dQ pass; the dK/dV pass is in
// fa_bwd_dkdv.h (its instantiations in fa_bwd_dkdv.hip and, for causal d = 128,
// fa_bwd_dkdv_ilp.hip, which is compiled with another instruction scheduler).
#include <type_traits>

#include "fa_bwd_common.h"

namespace fa {

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) and LSE * log2(e).  One thread per 8 elements of a row.
// The dQ pass can compute the same statistics itself (PRE): both sides form
// 8-element partial sums with chunk_dot and add them in one fixed tree, so the
// two give bitwise-identical D.
// ---------------------------------------------------------------------------
namespace {
// sum of the 8 products of two 16-byte chunks, in a fixed fma order
template <class T>
__device__ __forceinline__ float chunk_dot(const u32x4 &a, const u32x4 &b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc = __builtin_fmaf(T::lo(a[j]), T::lo(b[j]), acc);
    acc = __builtin_fmaf(T::hi(a[j]), T::hi(b[j]), acc);
  }
  return acc;
}
__device__ __forceinline__ float lse_log2(float l) {  // -inf: the row sees no key; +inf makes its P = 0
  return l == -__builtin_inff() ? __builtin_inff() : l * 1.4426950408889634f;
}
}  // namespace

template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ o,
                                                      const uint16_t *__restrict__ dout,
                                                      const float *__restrict__ lse,
                                                      float *__restrict__ dws,
                                                      float *__restrict__ lse2, long rows) {
  constexpr int TPR = D / 8;  // threads per row: chunk `sub` holds elements 8 sub .. 8 sub + 7
  const long row = (long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) acc = chunk_dot<T>(gload16(o + row * D + sub * 8), gload16(dout + row * D + sub * 8));
  // pairwise tree: chunks 8 apart (d = 128), 4, 2, then 1
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && sub == 0) {
    dws[row] = -acc;  // -D: the passes start their dP accumulation from it
    lse2[row] = lse_log2(lse[row]);
  }
}

// ---------------------------------------------------------------------------
// dQ: query-major pass
// ---------------------------------------------------------------------------
// PRE: the pass also computes D and LSE * log2(e) of its rows from O, dO and
// LSE and stores them for the dK/dV pass (no separate preprocessing kernel)
template <class T, int D, bool CAUSAL, bool DROP, bool PRE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BWD_DQ_OCC(D, DROP), BWD_DQ_OCC(D, DROP))))
void bwd_dq_kernel(BwdParams p) {
  constexpr int BN = 32;                // keys per step
  constexpr int BM = BWD_DQ_BM;         // query rows per workgroup (32 per wave)
  constexpr int RB = D * 2;             // bytes per tile row
  constexpr int TB = BN * RB;           // bytes per K (or V) tile
  constexpr int CPR = RB / 16;
  constexpr int ROWS_PER_BLOCK = 64 / CPR;
  constexpr int BPW = TB / 1024 / 4;    // DMA blocks per wave per tile
  constexpr int ND16 = D / 16, ND32 = D / 32;
  static_assert(BPW >= 1 && BM == 128, "tile shape");

  // K and V rings of NS slots, one LDS object per slot (the compiler can then
  // tell the slot being loaded from the slot being read); loads run NS - 1
  // steps ahead: three slots at d = 128 (cross-attention's backward 1.3 %
  // faster, square shapes unchanged), two at d = 64
  constexpr int NS = D == 128 ? BWD_DQ_NSLOT_D128 : 2;
  static_assert(NS == 2 || NS == 3, "two- or three-slot rings");
  __shared__ __attribute__((aligned(1024))) char k_slot0[TB];
  __shared__ __attribute__((aligned(1024))) char k_slot1[TB];
  __shared__ __attribute__((aligned(1024))) char k_slot2[NS == 3 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char v_slot0[TB];
  __shared__ __attribute__((aligned(1024))) char v_slot1[TB];
  __shared__ __attribute__((aligned(1024))) char v_slot2[NS == 3 ? TB : 16];
  constexpr int DMA_PER_STEP = 2 * BPW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, keep in an SGPR
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, s16 = lane & 15;

  int bh, qt;
  {
    const int nq = p.n_qtiles;
    int r;
    grid_tile((int)blockIdx.x, (int)gridDim.x / nq, nq, p.xcd_grouped, CAUSAL ? p.causal_group : 1, 0, bh, r);
    qt = CAUSAL ? nq - 1 - r : r;  // causal: longest rows first
  }
  const int i0 = qt * BM;
  const int wr0 = i0 + 32 * w;
  const int qrow = wr0 + l32;  // this lane's query
  // valid lengths of this batch entry; causal: query i sees keys j <= i + shift
  const int Nq = p.seq.Nq, Nk = p.seq.Nk;
  int Lq, Lk;
  seq_lengths(p.seq, bh / p.seq.H, Lq, Lk);
  const int shift = Lk - Lq;
  const size_t qoff = (size_t)bh * (size_t)Nq * D, koff = (size_t)bh * (size_t)Nk * D;
  // resources end at the valid rows: padding queries and keys read as zeros
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const uint16_t *>(p.q) + qoff, (uint32_t)Lq * RB);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(reinterpret_cast<const uint16_t *>(p.dout) + qoff, (uint32_t)Lq * RB);
  const char *k_head = reinterpret_cast<const char *>(p.k) + koff * 2;
  const char *v_head = reinterpret_cast<const char *>(p.v) + koff * 2;
  const uint32_t kv_bytes = (uint32_t)Lk * RB;

  const int kend = i0 >= Lq ? 0 : CAUSAL ? max(0, min(Lk, i0 + BM + shift)) : Lk;
  const int nt = (kend + BN - 1) / BN;
  const float sl2 = p.scale_log2;

  // per-lane row statistics; padding rows get lse2 = +inf so that P = 0
  const size_t srow = (size_t)bh * Nq + qrow;
  float lse2 = __builtin_inff(), ndsum = 0.f;  // ndsum = -D
  if constexpr (!PRE) {
    if (qrow < Lq) {
      lse2 = p.lse2[srow];
      ndsum = p.dws[srow];
    }
  }

  // Q and dO fragments: B operands of S^T = K Q^T and dP^T = V dO^T
  u32x4 qf[ND16], dof[ND16];
#pragma unroll
  for (int db = 0; db < ND16; ++db) {
    const uint32_t off = (uint32_t)(qrow * D + db * 16 + hi * 8) * 2;  // rows past Lq read 0
    qf[db] = bload16(rq, off);
    dof[db] = bload16(rdo, off);
  }

  if constexpr (PRE) {
    // this lane holds chunks 2 db + hi of its row's dO; the partial sums are
    // added in the preprocessing kernel's tree (chunks 8 apart, 4, 2, 1)
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(reinterpret_cast<const uint16_t *>(p.o) + qoff, (uint32_t)Lq * RB);
    float part[ND16];
#pragma unroll
    for (int db = 0; db < ND16; ++db)
      part[db] = chunk_dot<T>(bload16(ro, (uint32_t)(qrow * D + db * 16 + hi * 8) * 2), dof[db]);
    if constexpr (ND16 == 8) {
#pragma unroll
      for (int db = 0; db < 4; ++db) part[db] += part[db + 4];
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) part[db] += part[db + 2];
    float dsum = part[0] + part[1];
    dsum += __shfl_xor(dsum, 32);
    if (qrow < Lq) {
      lse2 = lse_log2(p.lse[srow]);
      ndsum = -dsum;
      if (hi == 0) {
        p.dws[srow] = ndsum;
        p.lse2[srow] = lse2;
      }
    }
  }

  // dP^T accumulates from -D (16 loop-invariant registers), so the MFMAs give
  // dP^T - D; with dropout dP is scaled first, and at d = 64 the registers are
  // not there (occupancy 4): both start from 0 and subtract
  constexpr bool DP_FROM_D = !DROP && D == 128;
  // K^T column blocks read before the softmax (d = 128 without dropout: the
  // other variants have no registers to spare)
  constexpr int KT_EARLY = DROP || D != 128 ? 0 : (BWD_DQ_KT_EARLY < ND32 ? BWD_DQ_KT_EARLY : ND32);
  f32x16 dp_init;
#pragma unroll
  for (int r = 0; r < 16; ++r) dp_init[r] = DP_FROM_D ? ndsum : 0.f;

  // K/V DMA into swizzled slots (K is read both ways, V only as fragments)
  uint32_t dk_off[BPW], dv_off[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int row = (w * BPW + j) * ROWS_PER_BLOCK + lane / CPR, pos = lane % CPR;
    dk_off[j] = (uint32_t)(row * RB + ((pos ^ swz_both<D>(row)) << 4));
    dv_off[j] = (uint32_t)(row * RB + ((pos ^ swz_frag<D>(row)) << 4));
  }
  // tile t goes to ring slot SL (tiles outside [0, nt) load as zeros)
  auto issue_step = [&](int t, auto slot) {
    constexpr int SL = decltype(slot)::value;
    // a resource per tile (scalar arithmetic): the per-lane offsets stay loop-invariant
    const bool ok = t >= 0 && t < nt;
    const __amdgpu_buffer_rsrc_t rkt = tile_rsrc(k_head, (uint32_t)t * TB, kv_bytes, ok);
    const __amdgpu_buffer_rsrc_t rvt = tile_rsrc(v_head, (uint32_t)t * TB, kv_bytes, ok);
    char *ks = SL == 0 ? k_slot0 : SL == 1 ? k_slot1 : k_slot2;
    char *vs = SL == 0 ? v_slot0 : SL == 1 ? v_slot1 : v_slot2;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      dma16(rkt, ks + (w * BPW + j) * 1024, dk_off[j]);
      dma16(rvt, vs + (w * BPW + j) * 1024, dv_off[j]);
    }
  };

  f32x16 dqacc[ND32];
#pragma unroll
  for (int c = 0; c < ND32; ++c) dqacc[c] = f32x16{};

  // Fragment-read byte offsets inside a slot: column block db of a K (V) row at
  // kf_base (vf_base) ^ (32 db); transposing reads of 32-column block c at
  // t_base[h] ^ (64 c), + 16 rows for the second half of the tile (the swizzles
  // permute whole 16-byte chunks of a row and repeat every 16 rows).
  uint32_t kf_base = (uint32_t)(l32 * RB + ((hi ^ swz_both<D>(l32)) << 4));
  uint32_t vf_base = (uint32_t)(l32 * RB + ((hi ^ swz_frag<D>(l32)) << 4));
  uint32_t t_base[2];
  {
    const int t_row = 4 * (g >> 1) + (s16 >> 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = t_row + 8 * h;
      const int byte = 32 * (g & 1) + 8 * (s16 & 3);
      t_base[h] = (uint32_t)(row * RB + (((byte >> 4) ^ swz_both<D>(row)) << 4) + (byte & 15));
    }
  }
  const int lim = CAUSAL ? min(qrow + shift, Lk - 1) : Lk - 1;  // last visible key

  // one step on key tile t held in ring slot SL
  auto step = [&](int t, auto slot) {
    constexpr int SL = decltype(slot)::value;
    issue_step(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
    const char *ks = SL == 0 ? k_slot0 : SL == 1 ? k_slot1 : k_slot2;
    const char *vs = SL == 0 ? v_slot0 : SL == 1 ? v_slot1 : v_slot2;
    // S^T = K Q^T and dP^T = V dO^T (keys x queries)
    f32x16 s = f32x16{}, dp = dp_init;
#pragma unroll
    for (int db = 0; db < ND16; ++db) {
      s = T::mma(lds_read16(ks + (kf_base ^ (uint32_t)(32 * db))), qf[db], s);
      dp = T::mma(lds_read16(vs + (vf_base ^ (uint32_t)(32 * db))), dof[db], dp);
    }
    // P^T = exp2(scale log2e S - LSE log2e), masked; dS^T = P^T (dP^T - D),
    // the difference already formed by the MFMAs
    // K^T operands of the first KT_EARLY column blocks of dQ^T += K^T dS^T,
    // read now: they do not depend on the softmax, and reads issued after the
    // mask branch could not be moved above it
    u32x4 kt[KT_EARLY > 0 ? KT_EARLY : 1][2];
#pragma unroll
    for (int c = 0; c < KT_EARLY; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const char *kk = ks + kb * 16 * RB;
        const u32x2 a0 = lds_read_tr4(kk + (t_base[0] ^ (uint32_t)(64 * c)));
        const u32x2 a1 = lds_read_tr4(kk + (t_base[1] ^ (uint32_t)(64 * c)));
        kt[c][kb] = u32x4{a0[0], a0[1], a1[0], a1[1]};
      }
    const int j0 = t * BN;
    const bool need_mask = (CAUSAL && j0 + BN - 1 > wr0 + shift) || (j0 + BN > Lk);
    // dropout: dP is masked and scaled (dS = P (Z dP - D), Z = keep * 256 / (256 - p8))
    const u32x4 keep = DROP ? keep_bytes_query_major(qrow, j0, hi, (uint32_t)bh, p.drop.offset, p.drop.k0, p.drop.k1)
                            : u32x4{};
    // masked tiles: the scores are scaled here and masked to -inf (so the mask
    // holds for any finite scale, zero and negative included), and the
    // exponent below multiplies by 1 instead of the scale
    if (need_mask) {  // a separate block: most steps skip it
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = key <= lim ? s[r] * sl2 : -__builtin_inff();
      }
    }
    const float mult = need_mask ? 1.f : sl2;
    uint32_t dsk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * j + e;
        const float pr = fast_exp2(__builtin_fmaf(s[r], mult, -lse2));  // masked: exp2(-inf) = 0
        if constexpr (DROP)
          v2[e] = pr * (kept(keep, r, p.drop.p8) ? __builtin_fmaf(dp[r], p.drop.scale, ndsum) : ndsum);
        else if constexpr (DP_FROM_D)
          v2[e] = pr * dp[r];
        else
          v2[e] = pr * (dp[r] + ndsum);
      }
      dsk[j] = T::pack(v2[0], v2[1]);
    }
    // dQ^T += K^T dS^T; K^T fragments by transposing reads of the K slot
#pragma unroll
    for (int c = 0; c < ND32; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 b = {dsk[4 * kb], dsk[4 * kb + 1], dsk[4 * kb + 2], dsk[4 * kb + 3]};
        if (c < KT_EARLY) {
          dqacc[c] = T::mma(kt[c < KT_EARLY ? c : 0][kb], b, dqacc[c]);
        } else {
          const char *kk = ks + kb * 16 * RB;
          const u32x2 a0 = lds_read_tr4(kk + (t_base[0] ^ (uint32_t)(64 * c)));
          const u32x2 a1 = lds_read_tr4(kk + (t_base[1] ^ (uint32_t)(64 * c)));
          dqacc[c] = T::mma(u32x4{a0[0], a0[1], a1[0], a1[1]}, b, dqacc[c]);
        }
      }
    }
    wait_vmcnt<(NS - 2) * DMA_PER_STEP>();  // tiles for step t + 1 have landed
    barrier_only();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2 % NS>;

  // a step on a key tile with no visible pair for this wave: only its share
  // of the loads and the barrier, which keep the workgroup's ring going
  auto idle_step = [&](int t, auto slot) {
    constexpr int SL = decltype(slot)::value;
    issue_step(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
    wait_vmcnt<(NS - 2) * DMA_PER_STEP>();
    barrier_only();
  };
  // causal: the key tiles from t_live on start past the last key this wave's
  // last row sees (they would add exact zeros to dQ); the lower waves of a
  // workgroup have up to three of them at the end of its range
  const int last_key = wr0 + 31 + shift;
  const int t_live = !CAUSAL ? nt : last_key < 0 ? 0 : min(nt, last_key / BN + 1);

  issue_step(0, S0{});
  if constexpr (NS == 3) issue_step(1, S1{});
  wait_vmcnt<(NS - 2) * DMA_PER_STEP>();
  barrier_only();
  int t = 0;
  for (; t + NS <= t_live; t += NS) {  // key tile t lives in slot t % NS
    step(t, S0{});
    step(t + 1, S1{});
    if constexpr (NS == 3) step(t + 2, S2{});
  }
  if (t < t_live) step(t, S0{});
  if constexpr (NS == 3) {
    if (t + 1 < t_live) step(t + 1, S1{});
  }
  for (int u = t_live; u < nt; ++u) {
    const int sl = u % NS;
    if (sl == 0)
      idle_step(u, S0{});
    else if (sl == 1)
      idle_step(u, S1{});
    else
      idle_step(u, S2{});
  }
  wait_vmcnt<0>();  // the trailing (zero-filled) loads have landed before exit

  // dQ = scale dQ^T^T, rounded to 16 bits (0 for padding rows), leaving
  // through LDS as whole rows (stage_put, stage_store_rows); the barrier: every wave's
  // trailing loads have landed in the ring, whose slots are free now
  barrier_only();
  static_assert(32 * RB <= TB, "a wave's dQ tile fits one ring slot");
  char *stage = w == 0 ? k_slot0 : w == 1 ? k_slot1 : w == 2 ? v_slot0 : v_slot1;
  const bool live = qrow < Lq;  // padding rows store zeros
  const float sc = p.scale;
#pragma unroll
  for (int c = 0; c < ND32; ++c)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      u32x2 st = {0u, 0u};
      if (live) {
        st[0] = T::pack(dqacc[c][4 * rg] * sc, dqacc[c][4 * rg + 1] * sc);
        st[1] = T::pack(dqacc[c][4 * rg + 2] * sc, dqacc[c][4 * rg + 3] * sc);
      }
      stage_put<D>(stage, c, rg, st, lane);
    }
  stage_store_rows<D>(stage, reinterpret_cast<uint16_t *>(p.dq) + qoff, wr0, Nq, lane);
}


// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <class T, int D>
static hipError_t launch_pre_t(const BwdParams &p, long rows, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);  // rows per workgroup
  const int grid = (int)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t *>(p.o),
                     reinterpret_cast<const uint16_t *>(p.dout), p.lse, p.dws, p.lse2, rows);
  return hipGetLastError();
}

template <class T, int D, bool C, bool PRE>
static hipError_t launch_dq_c(const BwdParams &p, int grid, hipStream_t st) {
  if (p.drop.p8 != 0)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, C, true, PRE>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, C, false, PRE>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}
template <class T, int D>
static hipError_t launch_dq_t(const BwdParams &p, int causal, int pre, int grid, hipStream_t st) {
  if (pre)
    return causal ? launch_dq_c<T, D, true, true>(p, grid, st) : launch_dq_c<T, D, false, true>(p, grid, st);
  return causal ? launch_dq_c<T, D, true, false>(p, grid, st) : launch_dq_c<T, D, false, false>(p, grid, st);
}

hipError_t launch_bwd_pre(const BwdParams &p, int dtype, int d, long rows, hipStream_t st) {
  if (dtype == 1) return d == 128 ? launch_pre_t<BF16, 128>(p, rows, st) : launch_pre_t<BF16, 64>(p, rows, st);
  return d == 128 ? launch_pre_t<F16, 128>(p, rows, st) : launch_pre_t<F16, 64>(p, rows, st);
}

hipError_t launch_bwd_dq(const BwdParams &p, int dtype, int d, int causal, int pre, int grid,
                         hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? launch_dq_t<BF16, 128>(p, causal, pre, grid, st)
                    : launch_dq_t<BF16, 64>(p, causal, pre, grid, st);
  return d == 128 ? launch_dq_t<F16, 128>(p, causal, pre, grid, st) : launch_dq_t<F16, 64>(p, causal, pre, grid, st);
}


}  // namespace fa
