// The dK/dV pass of the attention backward (key-major: one workgroup per 128
// keys, Q/dO tiles streamed through LDS; see fa_bwd.hip for the gradients and
// the orientation of the products).  Its instantiations live in
// fa_bwd_dkdv.hip and, for causal d = 128, in fa_bwd_dkdv_ilp.hip.
#pragma once

#include <type_traits>

#include "fa_bwd_common.h"

namespace fa {

// ---------------------------------------------------------------------------
// dK, dV: key-major pass
// ---------------------------------------------------------------------------
template <class T, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BWD_DKDV_OCC(D, DROP), BWD_DKDV_OCC(D, DROP))))
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BM = BWD_DKDV_BM;       // query rows per step
  constexpr int BN = BWD_DKDV_BN;       // keys per workgroup (32 per wave)
  constexpr int NS = BWD_DKDV_NSLOT;    // ring slots (loads run NS - 1 steps ahead)
  constexpr int RB = D * 2;
  constexpr int TB = BM * RB;           // bytes per Q (or dO) tile
  constexpr int STAT = BWD_DKDV_STAT;   // LSE2 (64 floats read, 32 used), then -D
  constexpr int SLOT = 2 * TB + STAT;   // Q, dO, stats
  constexpr int CPR = RB / 16;
  constexpr int ROWS_PER_BLOCK = 64 / CPR;
  constexpr int BPW = TB / 1024 / 4;
  constexpr int ND16 = D / 16, ND32 = D / 32;
  static_assert(BPW >= 1 && BM == 32 && BN == 128 && NS >= 2 && NS <= 3, "tile shape");
  // buffer->LDS loads a wave issues per step: Q and dO blocks, and (wave 0) the two stats rows
  constexpr int DMA_W = 2 * BPW, DMA_W0 = 2 * BPW + 2;

  // one LDS object per ring slot, so that the compiler can tell a slot being
  // loaded from the slot being read (it then needs no wait between the two)
  __shared__ __attribute__((aligned(1024))) char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) char slot2[NS == 3 ? SLOT : 16];
  auto slot_base = [&](auto slot) -> char * {
    constexpr int SL = decltype(slot)::value;
    if constexpr (SL == 0) return slot0;
    else if constexpr (SL == 1) return slot1;
    else return slot2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, keep in an SGPR
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, s16 = lane & 15;

  int bh, kt;
  {
    const int nk = p.n_ktiles;
    // causal: key tile 0 sees every query tile, so ascending order is heavy-first
    grid_tile((int)blockIdx.x, (int)gridDim.x / nk, nk, p.xcd_grouped, CAUSAL ? p.causal_group : 1, 0, bh, kt);
  }
  const int j0 = kt * BN;
  const int kw0 = j0 + 32 * w;
  const int key = kw0 + l32;  // this lane's key
  // valid lengths of this batch entry; causal: query i sees keys j <= i + shift
  const int Nq = p.seq.Nq, Nk = p.seq.Nk;
  int Lq, Lk;
  seq_lengths(p.seq, bh / p.seq.H, Lq, Lk);
  const int shift = Lk - Lq;
  const size_t qoff = (size_t)bh * (size_t)Nq * D, koff = (size_t)bh * (size_t)Nk * D;
  // resources end at the valid rows: padding rows read Q = dO = 0 and
  // LSE2 = D = 0 (so they add nothing to dK, dV), padding keys read K = V = 0
  const uint32_t q_bytes = (uint32_t)Lq * RB, k_bytes = (uint32_t)Lk * RB;
  const uint32_t stat_bytes = (uint32_t)Lq * 4;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const uint16_t *>(p.q) + qoff, q_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(reinterpret_cast<const uint16_t *>(p.dout) + qoff, q_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const uint16_t *>(p.k) + koff, k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const uint16_t *>(p.v) + koff, k_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse2 + (size_t)bh * Nq, stat_bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dws + (size_t)bh * Nq, stat_bytes);

  // K and V fragments of this wave's keys: B operands of S = Q K^T, dP = dO V^T
  u32x4 kf[ND16], vf[ND16];
#pragma unroll
  for (int db = 0; db < ND16; ++db) {
    const uint32_t off = (uint32_t)(key * D + db * 16 + hi * 8) * 2;  // keys past Lk read 0
    kf[db] = bload16(rk, off);
    vf[db] = bload16(rv, off);
  }
  // With dropout at d = 128 the last NVL V fragments live in LDS (one 16-byte
  // slot per thread, read back each step): the registers they free keep the
  // compiler from spilling, whose scratch reloads would wait on the tile DMA
  // in flight (both count in vmcnt) and so undo the prefetch.
  constexpr int NVL = DROP && D == 128 ? BWD_DKDV_DROP_VF_LDS : 0;
  __shared__ __attribute__((aligned(16))) u32x4 vf_lds[NVL > 0 ? NVL : 1][256];
#pragma unroll
  for (int j = 0; j < NVL; ++j) vf_lds[j][tid] = vf[ND16 - NVL + j];
  auto vfrag = [&](int db) -> u32x4 { return db >= ND16 - NVL ? vf_lds[db - (ND16 - NVL)][tid] : vf[db]; };

  // query tiles with valid rows that see a key of this block (none if all its keys are padding)
  const int nqt = j0 >= Lk ? 0 : (Lq + BM - 1) / BM;
  const int qt0 = CAUSAL ? max(0, j0 - shift) / BM : 0;
  const float sl2 = p.scale_log2;

  uint32_t dq_off[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int row = (w * BPW + j) * ROWS_PER_BLOCK + lane / CPR, pos = lane % CPR;
    dq_off[j] = (uint32_t)(row * RB + ((pos ^ swz_both<D>(row)) << 4));
  }
  // step i loads query tile qt0 + i into ring slot SL: Q, dO (swizzled), LSE2, D
  auto issue_step = [&](int i, auto slot) {
    const int qtile = qt0 + i;
    const bool ok = qtile < nqt;
    const uint32_t base = ok ? (uint32_t)qtile * TB : 0x80000000u;
    char *sp = slot_base(slot);
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      dma16(rq, sp + (w * BPW + j) * 1024, base + dq_off[j]);
      dma16(rdo, sp + TB + (w * BPW + j) * 1024, base + dq_off[j]);
    }
    if (w == 0) {  // 64 lanes x 4 bytes each: rows qtile*BM + lane (the first 32 are used)
      const uint32_t so = ok ? (uint32_t)(qtile * BM + lane) * 4 : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void *)(sp + 2 * TB), 4, so, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void *)(sp + 2 * TB + 256), 4, so, 0, 0, 0);
    }
  };
  // wait until at most `steps` steps of this wave's loads are in flight
  auto wait_dma = [&](auto steps) {
    constexpr int K = decltype(steps)::value;
    if (w == 0)
      wait_vmcnt<K * DMA_W0>();
    else
      wait_vmcnt<K * DMA_W>();
  };

  f32x16 dkacc[ND32], dvacc[ND32];
#pragma unroll
  for (int c = 0; c < ND32; ++c) {
    dkacc[c] = f32x16{};
    dvacc[c] = f32x16{};
  }

  // Fragment-read byte offsets inside a slot.  The 16-byte fragment of column
  // block db sits at f_base ^ (32 db): the swizzle permutes whole 16-byte chunks
  // of one row and 32 db only touches chunk bits.  Likewise the transposing
  // reads of 32-column block c sit at t_base[h] ^ (64 c), and the second
  // 16-row half of a tile at + 16 rows (the swizzles repeat every 16 rows).
  uint32_t f_base = (uint32_t)(l32 * RB + ((hi ^ swz_both<D>(l32)) << 4));
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

  // one step on query tile qt0 + i held in ring slot SL
  auto step = [&](int i, auto slot) {
    constexpr int SL = decltype(slot)::value;
    issue_step(i + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
    const char *qs = slot_base(slot);
    const char *ds = qs + TB;
    const float *ls = reinterpret_cast<const float *>(qs + 2 * TB);  // LSE2 at [0, 32), -D at [64, 96)
    const int q0 = (qt0 + i) * BM;
    // keep the per-block addresses out of the loop-invariant set: they are two
    // cheap VALU ops each, registers are not
    asm volatile("" : "+v"(f_base), "+v"(t_base[0]), "+v"(t_base[1]));
    // S = Q K^T and dP = dO V^T (queries x keys): lane = key, registers = queries.
    // dP accumulates from -D of each register's query row (the stats slot holds
    // -D at [64, 96)), so the MFMAs give dP - D; with dropout dP starts from 0
    f32x16 s = f32x16{}, dp;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4 nd = DROP ? f32x4{} : *reinterpret_cast<const f32x4 *>(ls + 64 + 8 * rg + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * rg + e] = nd[e];
    }
#pragma unroll
    for (int db = 0; db < ND16; ++db) {
      const uint32_t fa = f_base ^ (uint32_t)(32 * db);
      s = T::mma(lds_read16(qs + fa), kf[db], s);
      dp = T::mma(lds_read16(ds + fa), vfrag(db), dp);
    }
    const bool need_mask = CAUSAL && q0 + shift < kw0 + 31;
    // dropout: dV takes P * keep (scaled in the epilogue), dS = P (Z dP - D)
    const u32x4 keep = DROP ? keep_bytes_key_major(key, q0, hi, (uint32_t)bh, p.drop.offset, p.drop.k0, p.drop.k1)
                            : u32x4{};
    // masked tiles: scaled scores, -inf where masked; the exponent below then
    // multiplies by 1 instead of the scale (a mask that holds for any finite scale)
    if (need_mask) {  // a separate block: most steps skip it
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = key <= qrow + shift ? s[r] * sl2 : -__builtin_inff();
      }
    }
    const float mult = need_mask ? 1.f : sl2;
    // in two halves of 16 query rows (register groups 2kb, 2kb + 1): P and dS
    // packed to 16 bits, then dV^T += dO^T P and dK^T += Q^T dS for that half
    // (A operands by transposing reads); each accumulator still adds its kb = 0
    // product before its kb = 1 product
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t pk[4], sk[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rg = 2 * kb + h;
        const int qr = 8 * rg + 4 * hi;  // 4 consecutive query rows of this register group
        const f32x4 lq = *reinterpret_cast<const f32x4 *>(ls + qr);
        const f32x4 nd = DROP ? *reinterpret_cast<const f32x4 *>(ls + 64 + qr) : f32x4{};  // -D
        float pv[4], sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          // rows past Lq load LSE2 = D = 0 and Q = dO = 0, so they contribute nothing
          const float pr = fast_exp2(__builtin_fmaf(s[r], mult, -lq[e]));  // masked: exp2(-inf) = 0
          if constexpr (DROP) {
            const bool kp = kept(keep, r, p.drop.p8);
            pv[e] = kp ? pr : 0.f;
            sv[e] = pr * (kp ? __builtin_fmaf(dp[r], p.drop.scale, nd[e]) : nd[e]);
          } else {
            pv[e] = pr;
            sv[e] = pr * dp[r];  // dp already holds dP - D
          }
        }
        pk[2 * h] = T::pack(pv[0], pv[1]);
        pk[2 * h + 1] = T::pack(pv[2], pv[3]);
        sk[2 * h] = T::pack(sv[0], sv[1]);
        sk[2 * h + 1] = T::pack(sv[2], sv[3]);
      }
      const u32x4 bp = {pk[0], pk[1], pk[2], pk[3]};
      const u32x4 bs = {sk[0], sk[1], sk[2], sk[3]};
#pragma unroll
      for (int c = 0; c < ND32; ++c) {
        const uint32_t ta0 = t_base[0] ^ (uint32_t)(64 * c), ta1 = t_base[1] ^ (uint32_t)(64 * c);
        const u32x2 d0 = lds_read_tr4(ds + kb * 16 * RB + ta0);
        const u32x2 d1 = lds_read_tr4(ds + kb * 16 * RB + ta1);
        const u32x2 q0v = lds_read_tr4(qs + kb * 16 * RB + ta0);
        const u32x2 q1v = lds_read_tr4(qs + kb * 16 * RB + ta1);
        dvacc[c] = T::mma(u32x4{d0[0], d0[1], d1[0], d1[1]}, bp, dvacc[c]);
        dkacc[c] = T::mma(u32x4{q0v[0], q0v[1], q1v[0], q1v[1]}, bs, dkacc[c]);
      }
    }
    wait_dma(std::integral_constant<int, NS - 2>{});  // tiles for step i + 1 have landed
    barrier_only();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2 % NS>;

  // a step on a query tile with no visible pair for this wave: only its
  // share of the loads and the barrier, which keep the workgroup's ring going
  auto idle_step = [&](int i, auto slot) {
    constexpr int SL = decltype(slot)::value;
    issue_step(i + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
    wait_dma(std::integral_constant<int, NS - 2>{});
    barrier_only();
  };
  const int nsteps = max(0, nqt - qt0);
  // causal: the first i_live query tiles end before the first query that sees
  // this wave's first key (they would add exact zeros to dK and dV); wave w
  // of a workgroup on the diagonal has w of them
  int i_live = 0;
  if constexpr (CAUSAL) {
    const int need = kw0 - shift - (BM - 1);  // query tiles must reach this row
    i_live = need <= 0 ? 0 : min(nsteps, max(0, (need + BM - 1) / BM - qt0));
  }
  issue_step(0, S0{});
  if constexpr (NS == 3) issue_step(1, S1{});
  wait_dma(std::integral_constant<int, NS - 2>{});
  barrier_only();
  int i = 0;
  for (; i < i_live; ++i) {
    const int sl = i % NS;
    if (sl == 0)
      idle_step(i, S0{});
    else if (sl == 1)
      idle_step(i, S1{});
    else
      idle_step(i, S2{});
  }
  // live steps up to the next multiple of NS, where the unrolled loop's slots start
  if (i % NS == 1 && i < nsteps) step(i++, S1{});
  if constexpr (NS == 3) {
    if (i % NS == 2 && i < nsteps) step(i++, S2{});
  }
  for (; i + NS <= nsteps; i += NS) {  // query tile qt0 + i lives in slot i % NS
    step(i, S0{});
    step(i + 1, S1{});
    if constexpr (NS == 3) step(i + 2, S2{});
  }
  if (i < nsteps) step(i, S0{});
  if constexpr (NS == 3) {
    if (i + 1 < nsteps) step(i + 1, S1{});
  }
  wait_vmcnt<0>();  // the trailing (zero-filled) loads have landed before exit

  // dK = scale dK^T^T, dV = dV^T^T, rounded to 16 bits (0 for padding keys),
  // each leaving through LDS as whole rows (stage_put, stage_store_rows); the
  // barrier: every wave's trailing loads have landed in the ring, whose slots
  // are free now (two waves' tiles per slot).  With dropout the tiles are
  // stored directly (staged, the causal d = 128 kernel spilled under its
  // instruction scheduler).
  const bool live = key < Lk;  // padding keys store zeros (their sums are meaningless)
  const float sc = p.scale;
  const float sd = DROP ? p.drop.scale : 1.f;  // dV = sum (P * keep) dO * 256 / (256 - p8)
  if constexpr (!DROP) {
    barrier_only();
    static_assert(2 * 32 * RB <= SLOT, "two waves' tiles fit one ring slot");
    char *stage = (w < 2 ? slot0 : slot1) + (w & 1) * 32 * RB;
#pragma unroll
    for (int c = 0; c < ND32; ++c)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 st = {0u, 0u};
        if (live) {
          st[0] = T::pack(dkacc[c][4 * rg] * sc, dkacc[c][4 * rg + 1] * sc);
          st[1] = T::pack(dkacc[c][4 * rg + 2] * sc, dkacc[c][4 * rg + 3] * sc);
        }
        stage_put<D>(stage, c, rg, st, lane);
      }
    stage_store_rows<D>(stage, reinterpret_cast<uint16_t *>(p.dk) + koff, kw0, Nk, lane);
#pragma unroll
    for (int c = 0; c < ND32; ++c)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 st = {0u, 0u};
        if (live) {
          st[0] = T::pack(dvacc[c][4 * rg] * sd, dvacc[c][4 * rg + 1] * sd);
          st[1] = T::pack(dvacc[c][4 * rg + 2] * sd, dvacc[c][4 * rg + 3] * sd);
        }
        stage_put<D>(stage, c, rg, st, lane);
      }
    stage_store_rows<D>(stage, reinterpret_cast<uint16_t *>(p.dv) + koff, kw0, Nk, lane);
  } else if (key < Nk) {
    uint16_t *dKh = reinterpret_cast<uint16_t *>(p.dk) + koff;
    uint16_t *dVh = reinterpret_cast<uint16_t *>(p.dv) + koff;
#pragma unroll
    for (int c = 0; c < ND32; ++c)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int dcol = c * 32 + 8 * rg + 4 * hi;
        u32x2 a = {0u, 0u}, b = {0u, 0u};
        if (live) {
          a[0] = T::pack(dkacc[c][4 * rg] * sc, dkacc[c][4 * rg + 1] * sc);
          a[1] = T::pack(dkacc[c][4 * rg + 2] * sc, dkacc[c][4 * rg + 3] * sc);
          b[0] = T::pack(dvacc[c][4 * rg] * sd, dvacc[c][4 * rg + 1] * sd);
          b[1] = T::pack(dvacc[c][4 * rg + 2] * sd, dvacc[c][4 * rg + 3] * sd);
        }
        *reinterpret_cast<u32x2 *>(dKh + (size_t)key * D + dcol) = a;
        *reinterpret_cast<u32x2 *>(dVh + (size_t)key * D + dcol) = b;
      }
  }
}

template <class T, int D, bool C>
static hipError_t launch_dkdv_c(const BwdParams &p, int grid, hipStream_t st) {
  if (p.drop.p8 != 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, C, true>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, C, false>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

// causal d = 128 (fa_bwd_dkdv_ilp.hip)
hipError_t launch_bwd_dkdv_causal128(const BwdParams &p, int dtype, int grid, hipStream_t st);

}  // namespace fa
