// Attention backward for gfx950, with recomputation of the probabilities from
// the forward's log-sum-exp ("Flash Attention application", section
// "Recomputation": P is not stored, it is rebuilt in the backward; its v2
// section: the backward kernel's parallel schedule is what v2 reworked).
//
// Three kernels:
//   bwd_pre_kernel   D_i = sum_c dO_ic O_ic (fp32) and a zeroed fp32 dQ accumulator
//   bwd_kernel       one workgroup per (batch, head, 128-key tile); K_j and V_j stay
//                    in registers, query tiles of 64 rows stream through LDS:
//                      S = Q K_j^T, P = exp(scale S - LSE), dV_j += P^T dO,
//                      dP = dO V_j^T, dS = P (dP - D), dK_j += dS^T Q,
//                      dQ += dS K_j (fp32 atomics into the accumulator)
//   bwd_dq_kernel    dQ = scale * accumulator, rounded to 16 bits
// The gradient formulas are the calculus of O = softmax(scale Q K^T) V.
//
// MFMA orientation: S and dP are computed as [query][key] tiles (A = Q or dO
// fragments read from LDS, B = K^T or V^T fragments held in registers), so a
// lane owns one key (l % 32) and 16 queries.  P and dS packed to 16 bits are
// then directly the B operands of dV^T += dO^T P and dK^T += Q^T dS; the
// dO^T / Q^T A operands come from LDS through ds_read_b64_tr_b16.  dS is also
// written to LDS transposed ([key][query]) so that all four waves can form
// dQ = dS K over the workgroup's 128 keys.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) and zeroed dQ accumulator.  16 threads per row.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t *__restrict__ o,
                                                      const uint16_t *__restrict__ dout,
                                                      float *__restrict__ Dws,
                                                      float *__restrict__ dq_acc, long rows) {
  constexpr int TPR = 16;            // threads per row
  constexpr int EPT = D / TPR;       // elements per thread (8 or 4)
  const long row = (long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t *op = o + row * D + sub * EPT;
    const uint16_t *dp = dout + row * D + sub * EPT;
    if constexpr (EPT == 8) {
      const u32x4 a = gload16(op), b = gload16(dp);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += T::lo(a[j]) * T::lo(b[j]) + T::hi(a[j]) * T::hi(b[j]);
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2 *>(op), b = *reinterpret_cast<const u32x2 *>(dp);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc += T::lo(a[j]) * T::lo(b[j]) + T::hi(a[j]) * T::hi(b[j]);
    }
    float *qa = dq_acc + row * D + sub * EPT;
#pragma unroll
    for (int j = 0; j < EPT; j += 4) *reinterpret_cast<f32x4 *>(qa + j) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && sub == 0) Dws[row] = acc;
}

// ---------------------------------------------------------------------------
// dQ = scale * accumulator -> 16 bits.  4 elements per thread.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float *__restrict__ dq_acc,
                                                     uint16_t *__restrict__ dq, float scale,
                                                     long n4) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(dq_acc + 4 * i);
    u32x2 st;
    st[0] = T::pack(a[0] * scale, a[1] * scale);
    st[1] = T::pack(a[2] * scale, a[3] * scale);
    *reinterpret_cast<u32x2 *>(dq + 4 * i) = st;
  }
}

// ---------------------------------------------------------------------------
// main backward kernel
// ---------------------------------------------------------------------------
template <class T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_kernel(BwdParams p) {
  constexpr int BN = BWD_BN;          // keys per workgroup (32 per wave)
  constexpr int BM = BWD_BM;          // query rows per inner step
  constexpr int QS = D * 2 + 16;      // LDS row stride of Q / dO tiles (bytes)
  constexpr int KS = D * 2 + 64;      // LDS row stride of the K tile
  constexpr int SS = BM * 2 + 64;     // LDS row stride of the dS^T tile ([key][query])
  constexpr int QT = BM * QS;         // bytes of one Q (or dO) tile
  constexpr int STAGE = 2 * QT + 2 * BM * 4;  // Q, dO, LSE2, D
  constexpr int OFF_K = 2 * STAGE;
  constexpr int OFF_S = OFF_K + BN * KS;
  constexpr int LDS_BYTES = OFF_S + BN * SS;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int CPT = BM * CPR / 256; // chunks per thread per Q (or dO) tile
  constexpr int ND16 = D / 16, ND32 = D / 32, NQ32 = BM / 32, NQ16 = BM / 16;
  static_assert(BM * CPR % 256 == 0, "tile must split evenly over 256 threads");
  static_assert(BN == 128 && BM % 32 == 0, "tile shape");
  static_assert((BM / 32) * (D / 32) % 4 == 0, "dQ blocks must split evenly over 4 waves");

  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, s16 = lane & 15;
  const int N = p.N;

  int bh, kt;
  {
    const int nk = p.n_ktiles;
    const int bid = blockIdx.x;
    if (p.xcd_grouped) {
      const int x = bid & 7, kk = bid >> 3;
      bh = x + 8 * (kk / nk);
      kt = kk % nk;
    } else {
      bh = bid / nk;
      kt = bid % nk;
    }
    // causal: key tile 0 sees every query tile, so ascending order is heavy-first
  }
  const int j0 = kt * BN;
  const int kw0 = j0 + 32 * w;  // first key of this wave
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t *Qh = reinterpret_cast<const uint16_t *>(p.q) + hoff;
  const uint16_t *Kh = reinterpret_cast<const uint16_t *>(p.k) + hoff;
  const uint16_t *Vh = reinterpret_cast<const uint16_t *>(p.v) + hoff;
  const uint16_t *dOh = reinterpret_cast<const uint16_t *>(p.dout) + hoff;
  const float *Lh = p.lse + (size_t)bh * N;
  const float *Dh = p.dws + (size_t)bh * N;
  float *dQa = p.dq_acc + hoff;

  // ---- K, V fragments of this wave's 32 keys (B operands of Q K^T and dO V^T)
  u32x4 kf[ND16], vf[ND16];
  {
    const int key = kw0 + l32;
#pragma unroll
    for (int db = 0; db < ND16; ++db) {
      const size_t off = (size_t)key * D + db * 16 + hi * 8;
      kf[db] = key < N ? gload16(Kh + off) : u32x4{0, 0, 0, 0};
      vf[db] = key < N ? gload16(Vh + off) : u32x4{0, 0, 0, 0};
    }
  }
  // ---- the workgroup's K tile in LDS (B operand of dQ = dS K, transposing reads)
  {
    constexpr int KCPT = BN * CPR / 256;
#pragma unroll
    for (int c = 0; c < KCPT; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch / CPR, col = ch % CPR;
      const u32x4 val = j0 + row < N ? gload16(Kh + (size_t)(j0 + row) * D + col * 8) : u32x4{0, 0, 0, 0};
      lds_write16(smem + OFF_K + row * KS + col * 16, val);
    }
  }

  f32x16 dvacc[ND32], dkacc[ND32];
#pragma unroll
  for (int c = 0; c < ND32; ++c) {
    dvacc[c] = f32x16{};
    dkacc[c] = f32x16{};
  }

  const int nqt = (N + BM - 1) / BM;
  const int qt0 = CAUSAL ? j0 / BM : 0;
  const float sl2 = p.scale_log2;

  // ---- Q / dO tile staging: global -> registers -> LDS
  u32x4 pre[2 * CPT];
  float pre_l = 0.f, pre_d = 0.f;
  auto gfetch = [&](int qt) {
    const int q0 = qt * BM;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch / CPR, col = ch % CPR;
      const bool ok = q0 + row < N;
      const size_t off = (size_t)(q0 + row) * D + col * 8;
      pre[c] = ok ? gload16(Qh + off) : u32x4{0, 0, 0, 0};
      pre[CPT + c] = ok ? gload16(dOh + off) : u32x4{0, 0, 0, 0};
    }
    if (tid < BM) {
      const bool ok = q0 + tid < N;
      // rows past the end get LSE = +inf so that their P is exactly 0
      pre_l = ok ? Lh[q0 + tid] * 1.4426950408889634f : __builtin_inff();
      pre_d = ok ? Dh[q0 + tid] : 0.f;
    }
  };
  auto lstore = [&](int stage) {
    char *qs = smem + stage * STAGE;
    char *ds = qs + QT;
    float *ls = reinterpret_cast<float *>(qs + 2 * QT);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = tid + 256 * c;
      const int row = ch / CPR, col = ch % CPR;
      lds_write16(qs + row * QS + col * 16, pre[c]);
      lds_write16(ds + row * QS + col * 16, pre[CPT + c]);
    }
    if (tid < BM) {
      ls[tid] = pre_l;
      ls[BM + tid] = pre_d;
    }
  };

  gfetch(qt0);
  lstore(0);
  __syncthreads();

  char *sT = smem + OFF_S;  // dS^T tile, [key][query] 16-bit
  for (int qt = qt0; qt < nqt; ++qt) {
    const int it = qt - qt0;
    if (qt + 1 < nqt) gfetch(qt + 1);
    const char *qs = smem + (it & 1) * STAGE;
    const char *ds = qs + QT;
    const float *ls = reinterpret_cast<const float *>(qs + 2 * QT);
    const float *dsum = ls + BM;
    const int q0 = qt * BM;
    const bool active = !CAUSAL || q0 + BM - 1 >= kw0;
    if (active) {
      // -- S = Q K^T and dP = dO V^T, [query][key], NQ32 blocks of 32 queries
      f32x16 s[NQ32], dp[NQ32];
#pragma unroll
      for (int qb = 0; qb < NQ32; ++qb) {
        s[qb] = f32x16{};
        dp[qb] = f32x16{};
      }
#pragma unroll
      for (int db = 0; db < ND16; ++db)
#pragma unroll
        for (int qb = 0; qb < NQ32; ++qb) {
          const int off = (qb * 32 + l32) * QS + db * 32 + hi * 16;
          s[qb] = T::mma(lds_read16(qs + off), kf[db], s[qb]);
          dp[qb] = T::mma(lds_read16(ds + off), vf[db], dp[qb]);
        }
      // -- P = exp2(S scale log2e - LSE log2e), dS = P (dP - D); masked entries 0
      const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > N);
      const int key = kw0 + l32;
      uint32_t pk[NQ16][4], sk[NQ16][4];
#pragma unroll
      for (int qb = 0; qb < NQ32; ++qb) {
        float pv[16], dsv[16];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int qr = qb * 32 + 8 * rg + 4 * hi;  // 4 consecutive query rows
          const f32x4 lq = *reinterpret_cast<const f32x4 *>(ls + qr);
          const f32x4 dq = *reinterpret_cast<const f32x4 *>(dsum + qr);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            float pr = fast_exp2(__builtin_fmaf(s[qb][r], sl2, -lq[e]));
            if (need_mask) {
              const int qrow = q0 + qr + e;
              if ((CAUSAL && key > qrow) || key >= N) pr = 0.f;
            }
            pv[r] = pr;
            dsv[r] = pr * (dp[qb][r] - dq[e]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pk[qb * 2 + h][j] = T::pack(pv[8 * h + 2 * j], pv[8 * h + 2 * j + 1]);
            sk[qb * 2 + h][j] = T::pack(dsv[8 * h + 2 * j], dsv[8 * h + 2 * j + 1]);
          }
      }
      // -- dV^T += dO^T P and dK^T += Q^T dS (A operands by transposing LDS reads)
#pragma unroll
      for (int c = 0; c < ND32; ++c)
#pragma unroll
        for (int kb = 0; kb < NQ16; ++kb) {
          const int qrow = kb * 16 + 4 * (g >> 1) + (s16 >> 2);
          const int col = c * 32 + 16 * (g & 1) + 4 * (s16 & 3);
          const int off = qrow * QS + col * 2;
          const u32x2 d0 = lds_read_tr4(ds + off), d1 = lds_read_tr4(ds + off + 8 * QS);
          const u32x2 q0v = lds_read_tr4(qs + off), q1v = lds_read_tr4(qs + off + 8 * QS);
          const u32x4 ad = {d0[0], d0[1], d1[0], d1[1]};
          const u32x4 aq = {q0v[0], q0v[1], q1v[0], q1v[1]};
          const u32x4 bp = {pk[kb][0], pk[kb][1], pk[kb][2], pk[kb][3]};
          const u32x4 bs = {sk[kb][0], sk[kb][1], sk[kb][2], sk[kb][3]};
          dvacc[c] = T::mma(ad, bp, dvacc[c]);
          dkacc[c] = T::mma(aq, bs, dkacc[c]);
        }
      // -- dS^T to LDS: row = key (32 w + l32), 4 consecutive queries per write
#pragma unroll
      for (int kb = 0; kb < NQ16; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          // registers 8h..8h+7 of block qb hold queries qb*32 + 16h + 8*(j/4) + 4*hi + j%4
          const int qcol = kb * 16 + 8 * h2 + 4 * hi;
          u32x2 v2 = {sk[kb][2 * h2], sk[kb][2 * h2 + 1]};
          *reinterpret_cast<u32x2 *>(sT + (32 * w + l32) * SS + qcol * 2) = v2;
        }
    } else {
      // every query of this tile precedes every key of this wave: dS = 0
#pragma unroll
      for (int kb = 0; kb < NQ16; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int qcol = kb * 16 + 8 * h2 + 4 * hi;
          *reinterpret_cast<u32x2 *>(sT + (32 * w + l32) * SS + qcol * 2) = u32x2{0u, 0u};
        }
    }
    __syncthreads();
    // -- dQ[q][d] += sum_key dS[q][key] K[key][d] over the workgroup's keys; the
    //    (32-query, 32-column) blocks of the dQ tile are dealt round-robin to the waves
    if (!CAUSAL || q0 + BM - 1 >= j0) {
#pragma unroll
      for (int u = w; u < NQ32 * ND32; u += 4) {
        const int qb = u / ND32, c = u % ND32;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kb = 0; kb < BN / 16; ++kb) {
          // A = dS (query x key): rows of dS^T are keys -> transposing read
          const int krow = kb * 16 + 4 * (g >> 1) + (s16 >> 2);
          const int qcol = qb * 32 + 16 * (g & 1) + 4 * (s16 & 3);
          const char *ap = sT + krow * SS + qcol * 2;
          const u32x2 a0 = lds_read_tr4(ap), a1 = lds_read_tr4(ap + 8 * SS);
          // B = K (key x d): transposing read of the K tile
          const int dcol = 32 * c + 16 * (g & 1) + 4 * (s16 & 3);
          const char *bp = smem + OFF_K + krow * KS + dcol * 2;
          const u32x2 b0 = lds_read_tr4(bp), b1 = lds_read_tr4(bp + 8 * KS);
          acc = T::mma(u32x4{a0[0], a0[1], a1[0], a1[1]}, u32x4{b0[0], b0[1], b1[0], b1[1]}, acc);
        }
        // acc[r]: query qb*32 + 8*(r/4) + 4*hi + r%4, d column 32c + l32
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = q0 + qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (qrow < N) atomicAdd(dQa + (size_t)qrow * D + 32 * c + l32, acc[r]);
        }
      }
    }
    if (qt + 1 < nqt) lstore((it + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: dK = scale dK^T^T, dV = dV^T^T, rounded to 16 bits
  uint16_t *dKh = reinterpret_cast<uint16_t *>(p.dk) + hoff;
  uint16_t *dVh = reinterpret_cast<uint16_t *>(p.dv) + hoff;
  const int key = kw0 + l32;
  if (key < N) {
    const float sc = p.scale;
#pragma unroll
    for (int c = 0; c < ND32; ++c)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int dcol = c * 32 + 8 * rg + 4 * hi;
        u32x2 a, b;
        a[0] = T::pack(dkacc[c][4 * rg] * sc, dkacc[c][4 * rg + 1] * sc);
        a[1] = T::pack(dkacc[c][4 * rg + 2] * sc, dkacc[c][4 * rg + 3] * sc);
        b[0] = T::pack(dvacc[c][4 * rg], dvacc[c][4 * rg + 1]);
        b[1] = T::pack(dvacc[c][4 * rg + 2], dvacc[c][4 * rg + 3]);
        *reinterpret_cast<u32x2 *>(dKh + (size_t)key * D + dcol) = a;
        *reinterpret_cast<u32x2 *>(dVh + (size_t)key * D + dcol) = b;
      }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <class T, int D>
static hipError_t launch_pre_t(const BwdParams &p, long rows, hipStream_t st) {
  const int grid = (int)((rows + 15) / 16);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(grid), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t *>(p.o),
                     reinterpret_cast<const uint16_t *>(p.dout), p.dws, p.dq_acc, rows);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_main_t(const BwdParams &p, int causal, int grid, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((bwd_kernel<T, D, true>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_kernel<T, D, false>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_dq_t(const BwdParams &p, long elems, hipStream_t st) {
  const long n4 = elems / 4;
  hipLaunchKernelGGL((bwd_dq_kernel<T>), dim3((int)((n4 + 255) / 256)), dim3(256), 0, st,
                     p.dq_acc, reinterpret_cast<uint16_t *>(p.dq), p.scale, n4);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdParams &p, int dtype, int d, long rows, hipStream_t st) {
  if (dtype == 1) return d == 128 ? launch_pre_t<BF16, 128>(p, rows, st) : launch_pre_t<BF16, 64>(p, rows, st);
  return d == 128 ? launch_pre_t<F16, 128>(p, rows, st) : launch_pre_t<F16, 64>(p, rows, st);
}

hipError_t launch_bwd_main(const BwdParams &p, int dtype, int d, int causal, int grid,
                           hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? launch_main_t<BF16, 128>(p, causal, grid, st) : launch_main_t<BF16, 64>(p, causal, grid, st);
  return d == 128 ? launch_main_t<F16, 128>(p, causal, grid, st) : launch_main_t<F16, 64>(p, causal, grid, st);
}

hipError_t launch_bwd_dq(const BwdParams &p, int dtype, long elems, hipStream_t st) {
  return dtype == 1 ? launch_dq_t<BF16>(p, elems, st) : launch_dq_t<F16>(p, elems, st);
}

}  // namespace fa
