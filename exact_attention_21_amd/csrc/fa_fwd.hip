// Fused attention forward for gfx950.
//
// One workgroup = 4 waves = BM = 4 * 32 * QB query rows of one (batch, head);
// each wave owns 32 * QB rows.  The workgroup streams K/V tiles of BN keys
// through double-buffered LDS and runs the online softmax of the MHA tuning
// handbook ch.3 ("core idea": running max and running sum; "engineering
// implementation": per-block max, rescaling of the old partial output and sum,
// LSE kept per row).  Normalisation by the row sum happens once, in the
// epilogue, which is algebraically the same as the per-block division of that
// pseudocode.  Work partition follows the FA1-vs-FA2 page (section 2.1: each
// workgroup handles one query block, query fragments held in registers, K/V
// shared through on-chip memory; section 2.2: the next K/V tile is prefetched
// while the current one is computed).
//
// Scores are computed transposed, S^T = K Q^T, on 32x32x16 MFMAs: the A
// operand is a K fragment read from LDS, the B operand a Q fragment held in
// registers for the whole loop.  In the S^T accumulator a lane owns one query
// (l % 32) and 16 keys, so a row max/sum needs only in-lane reductions plus one
// exchange with the other half-wave.  The same registers, packed to 16 bits,
// are directly the B operand of O^T += V^T P^T; the V^T operand comes from LDS
// with the transposing read ds_read_b64_tr_b16.  Exponentials are base 2 with
// log2(e) folded into the score scale.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <class T, int D, int QB, int BN, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_kernel(FwdParams p) {
  constexpr int BM = 128 * QB;          // query rows per workgroup
  constexpr int WR = 32 * QB;           // query rows per wave
  constexpr int KS = D * 2 + 16;        // LDS row stride of K tiles (bytes)
  constexpr int VS = D * 2 + 64;        // LDS row stride of V tiles (bytes)
  constexpr int KT = BN * KS;           // bytes of one K tile
  constexpr int VT = BN * VS;           // bytes of one V tile
  constexpr int STAGE = KT + VT;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int CPT = BN * CPR / 256;   // chunks per thread per tile (K or V)
  constexpr int ND16 = D / 16, ND32 = D / 32, NK32 = BN / 32, NK16 = BN / 16;
  static_assert(BN * CPR % 256 == 0, "tile must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int N = p.N;

  // ---- which (head, query tile) this workgroup computes
  int bh, qt;
  {
    const int nq = p.n_qtiles;
    const int bid = blockIdx.x;
    int r;
    if (p.xcd_grouped) {  // heads of one XCD (bid % 8) run together: K/V stay in its L2
      const int x = bid & 7, kk = bid >> 3;
      bh = x + 8 * (kk / nq);
      r = kk % nq;
    } else {
      bh = bid / nq;
      r = bid % nq;
    }
    qt = CAUSAL ? nq - 1 - r : r;  // causal: longest rows first
  }
  const int i0 = qt * BM;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t *Qh = reinterpret_cast<const uint16_t *>(p.q) + hoff;
  const uint16_t *Kh = reinterpret_cast<const uint16_t *>(p.k) + hoff;
  const uint16_t *Vh = reinterpret_cast<const uint16_t *>(p.v) + hoff;

  const int wr0 = i0 + w * WR;  // first query row of this wave

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop
  u32x4 qf[QB][ND16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wr0 + qb * 32 + l32;
#pragma unroll
    for (int db = 0; db < ND16; ++db) {
      qf[qb][db] = row < N ? gload16(Qh + (size_t)row * D + db * 16 + hi * 8) : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 oacc[QB][ND32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int c = 0; c < ND32; ++c) oacc[qb][c] = f32x16{};
  float mrow[QB], lrow[QB];  // running max (log2 units) and this lane's partial sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -__builtin_inff();
    lrow[qb] = 0.f;
  }

  const int kend = CAUSAL ? min(N, i0 + BM) : N;
  const int ntiles = (kend + BN - 1) / BN;
  const float sl2 = p.scale_log2;

  // ---- K/V tile loading: global -> registers -> LDS (row-padded layout)
  u32x4 pre[2 * CPT];
  auto gfetch = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch / CPR, col = ch % CPR;
      const bool ok = j0 + row < N;
      const size_t off = (size_t)(j0 + row) * D + col * 8;
      pre[c] = ok ? gload16(Kh + off) : u32x4{0, 0, 0, 0};
      pre[CPT + c] = ok ? gload16(Vh + off) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int stage) {
    char *ks = smem + stage * STAGE;
    char *vs = ks + KT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch / CPR, col = ch % CPR;
      lds_write16(ks + row * KS + col * 16, pre[c]);
      lds_write16(vs + row * VS + col * 16, pre[CPT + c]);
    }
  };

  gfetch(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gfetch(t + 1);
    const char *ks = smem + (t & 1) * STAGE;
    const char *vs = ks + KT;
    const int j0 = t * BN;
    const bool active = !CAUSAL || j0 <= wr0 + WR - 1;
    if (active) {
      // -- S^T = K Q^T for BN keys x WR queries
      f32x16 s[NK32][QB];
#pragma unroll
      for (int kb = 0; kb < NK32; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int db = 0; db < ND16; ++db) {
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb) {
          const u32x4 a = lds_read16(ks + (kb * 32 + l32) * KS + db * 32 + hi * 16);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = T::mma(a, qf[qb][db], s[kb][qb]);
        }
      }
      // -- mask: causal diagonal tiles and the ragged tail of the keys
      const bool need_mask = (CAUSAL && j0 + BN - 1 > wr0) || (j0 + BN > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qrow = wr0 + qb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool masked = (CAUSAL && key > qrow) || key >= N;
              if (masked) s[kb][qb][r] = -__builtin_inff();
            }
          }
      }
      // -- online softmax: new running max, rescale factor, exponentials, row sum
      uint32_t pk[NK16][QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = max_xhalf(mx);
        const float mnew = fmaxf(mrow[qb], mx * sl2);
        const float mu = mnew == -__builtin_inff() ? 0.f : mnew;  // no (-inf) - (-inf)
        const float alpha = fast_exp2(mrow[qb] - mu);
        mrow[qb] = mnew;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(__builtin_fmaf(s[kb][qb][r], sl2, -mu));
            s[kb][qb][r] = e;
            ls += e;
          }
        lrow[qb] = lrow[qb] * alpha + ls;
#pragma unroll
        for (int c = 0; c < ND32; ++c) oacc[qb][c] *= alpha;
#pragma unroll
        for (int kb = 0; kb < NK32; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              pk[kb * 2 + h][qb][j] = T::pack(s[kb][qb][8 * h + 2 * j], s[kb][qb][8 * h + 2 * j + 1]);
      }
      // -- O^T += V^T P^T ; V^T fragments by transposing LDS reads
      const int g = lane >> 4, s16 = lane & 15;
#pragma unroll
      for (int c = 0; c < ND32; ++c) {
#pragma unroll
        for (int kb = 0; kb < NK16; ++kb) {
          const int krow = kb * 16 + 4 * (g >> 1) + (s16 >> 2);
          const int col = c * 32 + 16 * (g & 1) + 4 * (s16 & 3);
          const char *a0p = vs + krow * VS + col * 2;
          const u32x2 a0 = lds_read_tr4(a0p);
          const u32x2 a1 = lds_read_tr4(a0p + 8 * VS);
          const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const u32x4 b = {pk[kb][qb][0], pk[kb][qb][1], pk[kb][qb][2], pk[kb][qb][3]};
            oacc[qb][c] = T::mma(a, b, oacc[qb][c]);
          }
        }
      }
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (rounded to 16 bits), LSE = (m + log2 l) ln 2
  uint16_t *Oh = reinterpret_cast<uint16_t *>(p.o) + hoff;
  float *Lh = p.lse + (size_t)bh * N;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lrow[qb] + xhalf(lrow[qb]);
    const float inv = 1.f / lt;
    const int row = wr0 + qb * 32 + l32;
    if (row < N) {
#pragma unroll
      for (int c = 0; c < ND32; ++c)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int dcol = c * 32 + 8 * rg + 4 * hi;
          u32x2 st;
          st[0] = T::pack(oacc[qb][c][4 * rg + 0] * inv, oacc[qb][c][4 * rg + 1] * inv);
          st[1] = T::pack(oacc[qb][c][4 * rg + 2] * inv, oacc[qb][c][4 * rg + 3] * inv);
          *reinterpret_cast<u32x2 *>(Oh + (size_t)row * D + dcol) = st;
        }
      if (hi == 0) Lh[row] = (mrow[qb] + fast_log2(lt)) * 0.69314718055994531f;
    }
  }
}

// ---------------------------------------------------------------------------
// instantiation table
// ---------------------------------------------------------------------------

template <class T, int D, int QB, int BN, bool C>
static hipError_t launch_fwd_t(const FwdParams &p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<T, D, QB, BN, C>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams &p, int dtype, int d, int causal, int qb, int grid,
                      hipStream_t st) {
#define FA_FWD_CASE(TT, DD, QQ, BB)                                                   \
  if (d == DD && qb == QQ) {                                                          \
    return causal ? launch_fwd_t<TT, DD, QQ, BB, true>(p, grid, st)                   \
                  : launch_fwd_t<TT, DD, QQ, BB, false>(p, grid, st);                 \
  }
  if (dtype == 1) {
    FA_FWD_CASE(BF16, 128, 1, FWD_BN_D128)
    FA_FWD_CASE(BF16, 128, 2, FWD_BN_D128)
    FA_FWD_CASE(BF16, 64, 1, FWD_BN_D64)
    FA_FWD_CASE(BF16, 64, 2, FWD_BN_D64)
  } else {
    FA_FWD_CASE(F16, 128, 1, FWD_BN_D128)
    FA_FWD_CASE(F16, 128, 2, FWD_BN_D128)
    FA_FWD_CASE(F16, 64, 1, FWD_BN_D64)
    FA_FWD_CASE(F16, 64, 2, FWD_BN_D64)
  }
#undef FA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
