// Fused attention forward for gfx950.
//
// One workgroup = 4 waves = BM = 128 * QB query rows of one (batch, head); each
// wave owns 32 * QB rows.  The workgroup streams K/V tiles of BN = 32 keys
// through LDS and runs the online softmax of the MHA tuning handbook ch.3
// ("core idea": running max and running sum; "engineering implementation":
// per-block max, rescaling of the old partial output and sum, LSE kept per
// row).  Normalisation by the row sum happens once, in the epilogue, which is
// algebraically the same as that pseudocode's per-block division.  Work
// partition follows the FA1-vs-FA2 page (section 2.1: each workgroup handles one
// query block with its query fragments held in registers and K/V shared
// through on-chip memory; section 2.2: later K/V tiles are fetched while the
// current one is computed).
//
// Scores are computed transposed, S^T = K Q^T, on 32x32x16 MFMAs: the A operand
// is a K fragment read from LDS, the B operand a Q fragment held in registers
// for the whole loop.  In the S^T accumulator a lane owns one query (l % 32)
// and 16 keys, so a row max/sum needs in-lane reductions plus one exchange with
// the other half-wave.  The same registers, packed to 16 bits, are directly the
// B operand of O^T += V^T P^T; the V^T operand comes from LDS through the
// transposing read ds_read_b64_tr_b16.  Exponentials are base 2 with log2(e)
// folded into the score scale.
//
// K/V tiles reach LDS by direct buffer->LDS loads (no staging registers) into
// rings of two or three slots, one or two steps ahead (one LDS object per
// slot, so that the compiler sees the load into one slot and the reads of the
// others do not alias); each tile's buffer resource starts at the tile, so the
// per-lane load offsets stay loop-invariant.  Tiles are stored with unpadded rows and an XOR swizzle of the
// 16-byte chunk index chosen per access pattern (K: chunk ^ (row & 15) at
// d = 128, conflict-free for the 16-byte fragment reads; V: a swizzle of row
// bits 0..3 conflict-free for the transposing reads).  Rows past the valid
// length load as zeros (hardware range check of the buffer resource).
//
// One kernel serves the square, padded / cross-attention, dropout and
// split-over-keys entry points: per batch entry it reads the valid lengths Lq,
// Lk and shifts the causal limit by Lk - Lq; DROP adds the Philox keep bits to
// P; SPLIT restricts the workgroup to one chunk of keys and writes fp32
// partials for the merge kernel below.
//
// Latency is hidden by occupancy rather than by software pipelining: the kernel
// fits in 168 VGPRs, so three workgroups (12 waves) share a CU and the
// sequencer interleaves one wave's exponentials with another's MFMAs.  Each
// row's running max is raised lazily: only when the row's max grows by more
// than 2^8 are its running max, row sum and output row rescaled (the output
// rescale is a wave-uniform, rarely taken branch).  Between raises the
// exponentials are taken against a stale max, so p <= 2^8; the final
// normalisation uses the same stale max in numerator and denominator, so the
// result is unchanged.  A tile's row max is only needed when some p would
// exceed 2^8, so each tile first takes the exponentials against the running
// max and checks every lane's partial row sum against 2^8; only a wave in
// which a sum exceeds it (a row's first visible tile always does) computes the
// row max, updates and takes the exponentials again.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float LAZY_TAU = 8.0f;  // log2 growth of a row max that forces a rescale
constexpr float LAZY_BOUND = 256.0f;  // 2^LAZY_TAU: largest probability kept without a rescale
constexpr float M_FLOOR = -1e30f; // initial running max (log2 units)

// XOR swizzles of the 16-byte chunk index within a tile row.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// The V swizzle depends on row bits 0..3 only: the fragment reads add 16 rows
// to a precomputed address for the second 16-key half of a tile.
template <int D>
__host__ __device__ constexpr int swz_v(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row & 3) << 1) ^ ((row >> 2) & 3)) & 7);
}
template <int D>
constexpr bool swz_v_period16() {
  for (int r = 0; r < 16; ++r)
    if (swz_v<D>(r + 16) != swz_v<D>(r)) return false;
  return true;
}
static_assert(swz_v_period16<64>() && swz_v_period16<128>(), "V swizzle must repeat every 16 rows");

}  // namespace

// waves per SIMD: two query blocks per wave need the registers of occupancy 2
#define FWD_OCC(D, QB, DROP) ((QB) == 2 ? 2 : (D) == 64 ? FWD_WAVES_D64 : FWD_WAVES_PER_SIMD)

template <class T, int D, int QB, bool CAUSAL, bool DROP, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FWD_OCC(D, QB, DROP), FWD_OCC(D, QB, DROP))))
void fwd_kernel(FwdParams p) {
  constexpr int BN = FWD_BN;
  constexpr int BM = 128 * QB;          // query rows per workgroup
  constexpr int WR = 32 * QB;           // query rows per wave
  constexpr int RB = D * 2;             // bytes per tile row (unpadded)
  constexpr int TB = BN * RB;           // bytes of one K (or V) tile
  constexpr int CPR = RB / 16;          // 16-byte chunks per row
  constexpr int ROWS_PER_BLOCK = 64 / CPR;       // rows covered by one 1 KB DMA block
  constexpr int BLOCKS = TB / 1024;              // DMA blocks per tile
  constexpr int BPW = BLOCKS / 4;                // DMA blocks per wave per tile
  constexpr int ND16 = D / 16, ND32 = D / 32;
  static_assert(BLOCKS % 4 == 0, "tile must split evenly over 4 waves");

  // K and V rings of NS slots, one LDS object per slot (the compiler can then
  // tell the slot being loaded from the slot being read).  Tiles are loaded
  // NS - 1 steps ahead: three slots for the split forward (decode shapes, bound
  // by how many bytes are in flight to HBM) and for d = 128 (cross-attention
  // and ragged batches gain 3-4 %, square causal shapes ~0.5 %), two at d = 64
  // and with dropout (three measured 2-4 % slower there).
  constexpr int NS = SPLIT ? FWD_NSLOT_SPLIT : (D == 128 && !DROP ? FWD_NSLOT_D128 : 2);
  static_assert(NS == 2 || NS == 3, "two- or three-slot rings");
  __shared__ __attribute__((aligned(1024))) char k_slot0[TB];
  __shared__ __attribute__((aligned(1024))) char k_slot1[TB];
  __shared__ __attribute__((aligned(1024))) char k_slot2[NS == 3 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char v_slot0[TB];
  __shared__ __attribute__((aligned(1024))) char v_slot1[TB];
  __shared__ __attribute__((aligned(1024))) char v_slot2[NS == 3 ? TB : 16];
  auto kslot = [&](auto slot) -> char * {
    constexpr int SL = decltype(slot)::value;
    return SL == 0 ? k_slot0 : SL == 1 ? k_slot1 : k_slot2;
  };
  auto vslot = [&](auto slot) -> char * {
    constexpr int SL = decltype(slot)::value;
    return SL == 0 ? v_slot0 : SL == 1 ? v_slot1 : v_slot2;
  };
  constexpr int DMA_PER_STEP = 2 * (TB / 1024 / 4);  // K and V blocks one wave loads per step

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, keep in an SGPR
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = lane >> 4, s16 = lane & 15;

  // ---- which (head, query tile) this workgroup computes
  static_assert(!(SPLIT && DROP), "the split forward has no dropout");
  int bh, qt;
  const int split = SPLIT ? (int)(blockIdx.x % (unsigned)p.nsplit) : 0;
  {
    const int nq = p.n_qtiles;
    const int bid = SPLIT ? (int)(blockIdx.x / (unsigned)p.nsplit) : (int)blockIdx.x;
    const int heads = (int)(gridDim.x / (SPLIT ? (unsigned)p.nsplit : 1u)) / nq;
    int r;
    // causal: heads in groups of p.causal_group, and the last heads (two rounds of the FWD_OCC
    // workgroups per CU of an XCD's 32 CUs, or of all 256 when the heads are
    // not grouped per XCD) in one group, so that the grid ends on short tiles
    grid_tile(bid, heads, nq, p.xcd_grouped, CAUSAL ? p.causal_group : 1,
              CAUSAL ? causal_tail_heads(nq, (p.xcd_grouped ? 32 : 256) * FWD_OCC(D, QB, DROP)) : 0, bh, r);
    qt = CAUSAL ? nq - 1 - r : r;  // causal: longest rows first
  }
  const int i0 = qt * BM;
  // valid lengths of this batch entry; causal: query i sees keys j <= i + shift
  const int Nq = p.seq.Nq, Nk = p.seq.Nk;
  int Lq, Lk;
  seq_lengths(p.seq, bh / p.seq.H, Lq, Lk);
  const int shift = Lk - Lq;
  const size_t qoff = (size_t)bh * (size_t)Nq * D, koff = (size_t)bh * (size_t)Nk * D;
  // resources end at the valid rows: padding queries (and keys, below) read as zeros
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const uint16_t *>(p.q) + qoff, (uint32_t)Lq * RB);
  const int wr0 = i0 + w * WR;  // first query row of this wave

  // keys the workgroup's rows can see (none if all its rows are padding)
  const int kend = i0 >= Lq ? 0 : CAUSAL ? max(0, min(Lk, i0 + BM + shift)) : Lk;
  const int nt = (kend + BN - 1) / BN;
  // key tiles of this workgroup: all of them, or one chunk of the split forward
  const int t_beg = SPLIT ? min(nt, split * (p.chunk / BN)) : 0;
  const int t_end = SPLIT ? min(nt, t_beg + p.chunk / BN) : nt;
  const float sl2 = p.scale_log2;

  // ---- K/V tile DMA: this lane's share of block (w * BPW + j) of a tile
  uint32_t dma_k_off[BPW], dma_v_off[BPW];  // byte offset inside a tile (swizzled source)
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int blk = w * BPW + j;
    const int row = blk * ROWS_PER_BLOCK + lane / CPR, pos = lane % CPR;
    dma_k_off[j] = (uint32_t)(row * RB + ((pos ^ swz_k<D>(row)) << 4));
    dma_v_off[j] = (uint32_t)(row * RB + ((pos ^ swz_v<D>(row)) << 4));
  }
  // Each tile gets a buffer resource of its own (scalar arithmetic), so the
  // per-lane offsets stay loop-invariant: the resource starts at the tile and
  // ends at the valid keys; tiles outside [t_beg, t_end) get zero records and
  // load as zeros.
  const char *k_head = reinterpret_cast<const char *>(p.k) + koff * 2;
  const char *v_head = reinterpret_cast<const char *>(p.v) + koff * 2;
  const uint32_t kv_bytes = (uint32_t)Lk * RB;
  auto issue_tile = [&](const char *head, int t, char *slot, const uint32_t (&offs)[BPW]) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(head, (uint32_t)t * TB, kv_bytes, t >= t_beg && t < t_end);
#pragma unroll
    for (int j = 0; j < BPW; ++j) dma16(r, slot + (w * BPW + j) * 1024, offs[j]);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop
  u32x4 qf[QB][ND16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wr0 + qb * 32 + l32;  // rows past Lq read as zeros
#pragma unroll
    for (int db = 0; db < ND16; ++db)
      qf[qb][db] = bload16(rq, (uint32_t)(row * D + db * 16 + hi * 8) * 2);
  }

  f32x16 oacc[QB][ND32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int c = 0; c < ND32; ++c) oacc[qb][c] = f32x16{};
  float mrun[QB], lrun[QB];  // running max (log2 units) and this lane's partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // a finite floor instead of -inf: a row that sees no key in a tile then
    // takes exp2(-inf - floor) = 0 rather than exp2(-inf + inf) = NaN, and
    // the first visible tile always raises the max (alpha = exp2(floor - m) = 0)
    mrun[qb] = M_FLOOR;
    lrun[qb] = 0.f;
  }

  f32x16 sacc[QB];
  uint32_t pk[QB][8];

  // fragment-read byte offsets inside a slot, computed once (the slot base is a
  // compile-time constant in the two-way unrolled loop below)
  uint32_t k_addr[ND16];
#pragma unroll
  for (int db = 0; db < ND16; ++db)
    k_addr[db] = (uint32_t)(l32 * RB + (((2 * db + hi) ^ swz_k<D>(l32)) << 4));
  uint32_t v_addr[ND32][2];  // [32-column block][first / second 4-row read]
  {
    const int v_row = 4 * (g >> 1) + (s16 >> 2);  // + 16 kb for the second 16-key half
#pragma unroll
    for (int c = 0; c < ND32; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = v_row + 8 * h;  // swz_v(row + 16) == swz_v(row)
        const int byte = c * 64 + 32 * (g & 1) + 8 * (s16 & 3);
        v_addr[c][h] = (uint32_t)(row * RB + (((byte >> 4) ^ swz_v<D>(row)) << 4) + (byte & 15));
      }
  }

  // S(t) = K(t) Q^T, K(t) in ring slot SL
  auto stage_s = [&](auto slot, f32x16 (&s)[QB]) {
    const char *ks = kslot(slot);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
    for (int db = 0; db < ND16; ++db) {
      const u32x4 a = lds_read16(ks + k_addr[db]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = T::mma(a, qf[qb][db], s[qb]);
    }
  };
  // masking of tile t: causal diagonal and the ragged key tail
  auto needs_mask = [&](int t) {
    const int j0 = t * BN;
    return (CAUSAL && j0 + BN - 1 > wr0 + shift) || (j0 + BN > Lk);
  };
  // The mask is applied to the scaled scores (scale * log2(e) * s, or -inf),
  // so that it holds for any finite scale, zero and negative included; the
  // softmax of a masked tile then multiplies by 1 instead of the scale.
  auto apply_mask = [&](int t, f32x16 (&s)[QB]) {
    const int j0 = t * BN;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = wr0 + qb * 32 + l32;
      const int lim = CAUSAL ? min(qrow + shift, Lk - 1) : Lk - 1;  // last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[qb][r] = key <= lim ? s[qb][r] * sl2 : -__builtin_inff();
      }
    }
  };
  // probabilities p = exp2(s * mult - m) of one block against the reference
  // max m (mult = scale * log2(e), or 1 for a masked tile whose scores are
  // already scaled), packed to 16 bits (dropout-masked), and this lane's share
  // of the row sum, taken from the unrounded, unmasked values
  auto probs = [&](const f32x16 &s, float mult, float m, uint32_t (&pk)[8], const u32x4 &keep) {
    const float nm = -m;
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e0 = fast_exp2(__builtin_fmaf(s[2 * j], mult, nm));
      const float e1 = fast_exp2(__builtin_fmaf(s[2 * j + 1], mult, nm));
      if constexpr (DROP)  // dropped weights leave P V but not the row sum
        pk[j] = T::pack(kept(keep, 2 * j, p.drop.p8) ? e0 : 0.f, kept(keep, 2 * j + 1, p.drop.p8) ? e1 : 0.f);
      else
        pk[j] = T::pack(e0, e1);
      ls = j == 0 ? e0 + e1 : ls + (e0 + e1);
    }
    return ls;
  };
  // softmax of one tile; returns whether a running max moved (the output must
  // be rescaled).  Fast path: the probabilities against the current running
  // max are final when none exceeds 2^tau, which a lane's partial row sum
  // <= 2^tau guarantees (the sum is +inf on a row's first visible tile, whose
  // running max is still the floor, and NaN fails the test too).  Otherwise,
  // for the whole wave: the lazy update of the running max from the tile's row
  // max, and the probabilities again.
  auto stage_softmax = [&](f32x16 (&s)[QB], float mult, uint32_t (&pk)[QB][8], float (&alpha)[QB],
                           const u32x4 (&keep)[QB]) {
    float ls[QB];
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ls[qb] = probs(s[qb], mult, mrun[qb], pk[qb], keep[qb]);
      over |= !(ls[qb] <= LAZY_BOUND);
    }
    if (__builtin_amdgcn_ballot_w64(over) == 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        alpha[qb] = 1.f;
        lrun[qb] += ls[qb];
      }
      return false;
    }
    bool grow_any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // row max of the scaled scores (the products, so that a negative scale
      // takes the smallest raw score)
      float mx = fmaxf(s[qb][0] * mult, s[qb][1] * mult);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[qb][r] * mult, s[qb][r + 1] * mult));
      mx = max_xhalf(mx);
      // per-row lazy update (a lane-wise select, not a branch)
      const bool grow = mx > mrun[qb] + LAZY_TAU;
      const float mu = grow ? mx : mrun[qb];
      alpha[qb] = grow ? fast_exp2(mrun[qb] - mx) : 1.f;
      grow_any |= grow;
      mrun[qb] = mu;
      lrun[qb] = lrun[qb] * alpha[qb] + probs(s[qb], mult, mu, pk[qb], keep[qb]);
    }
    return grow_any;
  };
  // O^T += V(t)^T P(t)^T, V(t) in ring slot SL; the 16-key halves outermost, so
  // that consecutive MFMAs share their B operand (each output block still adds
  // its first half before its second)
  auto stage_pv = [&](auto slot, const uint32_t (&pk)[QB][8]) {
    const char *vs = vslot(slot);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int c = 0; c < ND32; ++c) {
        const u32x2 a0 = lds_read_tr4(vs + kb * 16 * RB + v_addr[c][0]);
        const u32x2 a1 = lds_read_tr4(vs + kb * 16 * RB + v_addr[c][1]);
        const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const u32x4 b = {pk[qb][4 * kb], pk[qb][4 * kb + 1], pk[qb][4 * kb + 2], pk[qb][4 * kb + 3]};
          oacc[qb][c] = T::mma(a, b, oacc[qb][c]);
        }
      }
    }
  };
  auto rescale_o = [&](const float (&alpha)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int c = 0; c < ND32; ++c) oacc[qb][c] *= alpha[qb];
  };

  // K(t) and V(t) go to ring slot SL
  auto issue_step = [&](int t, auto slot) {
    issue_tile(k_head, t, kslot(slot), dma_k_off);
    issue_tile(v_head, t, vslot(slot), dma_v_off);
  };
  // one step on tile t held in slot SL; tile t + NS - 1 is loaded into its slot
  auto step = [&](int t, auto slot) {
    constexpr int SL = decltype(slot)::value;
    issue_step(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
    stage_s(slot, sacc);
    // dropout bytes of this lane's 16 pairs per query block (generated after
    // the S MFMAs are issued: fewer registers live across them)
    u32x4 keep[QB] = {};
    if constexpr (DROP) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        keep[qb] = keep_bytes_query_major(wr0 + qb * 32 + l32, t * BN, hi, (uint32_t)bh, p.drop.offset,
                                          p.drop.k0, p.drop.k1);
    }
    const bool masked = needs_mask(t);
    if (masked) apply_mask(t, sacc);
    float alpha[QB];
    const bool resc = stage_softmax(sacc, masked ? 1.f : sl2, pk, alpha, keep);
    if (__builtin_amdgcn_ballot_w64(resc) != 0) rescale_o(alpha);
    stage_pv(slot, pk);
    wait_vmcnt<(NS - 2) * DMA_PER_STEP>();  // tiles for step t + 1 have landed
    barrier_only();
  };
  // a step on a tile with no visible pair for this wave: only its share of
  // the loads and the barrier, which keep the workgroup's ring going
  auto idle_step = [&](int t, auto slot) {
    constexpr int SL = decltype(slot)::value;
    issue_step(t + NS - 1, std::integral_constant<int, (SL + NS - 1) % NS>{});
    wait_vmcnt<(NS - 2) * DMA_PER_STEP>();
    barrier_only();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  using S2 = std::integral_constant<int, 2 % NS>;

  // causal: the tiles from t_live on start past the last key this wave's
  // last row sees (their softmax would add exact zeros); the lower waves of
  // a workgroup have up to three of them at the end of its range
  const int last_key = wr0 + QB * 32 - 1 + shift;
  const int t_live = !CAUSAL ? t_end : last_key < 0 ? t_beg : max(t_beg, min(t_end, last_key / BN + 1));

  issue_step(t_beg, S0{});
  if constexpr (NS == 3) issue_step(t_beg + 1, S1{});
  wait_vmcnt<(NS - 2) * DMA_PER_STEP>();
  barrier_only();
  int t = t_beg;
  for (; t + NS <= t_live; t += NS) {  // tile t lives in slot (t - t_beg) % NS
    step(t, S0{});
    step(t + 1, S1{});
    if constexpr (NS == 3) step(t + 2, S2{});
  }
  if (t < t_live) step(t, S0{});
  if constexpr (NS == 3) {
    if (t + 1 < t_live) step(t + 1, S1{});
  }
  for (int u = t_live; u < t_end; ++u) {
    const int sl = (u - t_beg) % NS;
    if (sl == 0)
      idle_step(u, S0{});
    else if (sl == 1)
      idle_step(u, S1{});
    else
      idle_step(u, S2{});
  }
  wait_vmcnt<0>();  // the trailing (zero-filled) loads have landed before exit

  // ---- epilogue: O = acc / l (rounded to 16 bits), LSE = (m + log2 l) ln 2;
  // the split forward writes this chunk's O (fp32) and LSE to the partials
  uint16_t *Oh = reinterpret_cast<uint16_t *>(p.o) + qoff;
  float *Lh = p.lse + (size_t)bh * Nq;
  const size_t pbase = SPLIT ? ((size_t)bh * p.nsplit + split) * Nq : 0;
  if constexpr (!SPLIT && QB == 1) {
    // O leaves through LDS as whole rows (stage_put, stage_store_rows); the barrier:
    // every wave's trailing loads have landed in the ring, whose slots are
    // free now (one per wave)
    barrier_only();
    static_assert(32 * RB <= TB, "a wave's output tile fits one ring slot");
    char *stage = w == 0 ? k_slot0 : w == 1 ? k_slot1 : w == 2 ? v_slot0 : v_slot1;
    const float lt = lrun[0] + xhalf(lrun[0]);
    const int row = wr0 + l32;
    // padding rows and rows that see no key (row sum exactly 0): O = 0,
    // LSE = -inf; a live row's sum is >= 1 (its largest term is taken against
    // a running max no larger than the row's max), and NaN stays NaN
    const bool live = row < Lq && lt != 0.f;
    const float inv = (DROP ? p.drop.scale : 1.f) / lt;  // kept weights are scaled by 256 / (256 - p8)
#pragma unroll
    for (int c = 0; c < ND32; ++c)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 st = {0u, 0u};
        if (live) {
          st[0] = T::pack(oacc[0][c][4 * rg + 0] * inv, oacc[0][c][4 * rg + 1] * inv);
          st[1] = T::pack(oacc[0][c][4 * rg + 2] * inv, oacc[0][c][4 * rg + 3] * inv);
        }
        stage_put<D>(stage, c, rg, st, lane);
      }
    if (hi == 0 && row < Nq) Lh[row] = live ? (mrun[0] + fast_log2(lt)) * 0.69314718055994531f : -__builtin_inff();
    stage_store_rows<D>(stage, Oh, wr0, Nq, lane);
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = lrun[qb] + xhalf(lrun[qb]);
      const int row = wr0 + qb * 32 + l32;
      // padding rows and rows that see no key (row sum exactly 0): O = 0,
      // LSE = -inf; a live row's sum is >= 1 (its largest term is taken against
      // a running max no larger than the row's max), and NaN stays NaN
      const bool live = row < Lq && lt != 0.f;
      const float inv = (DROP ? p.drop.scale : 1.f) / lt;  // kept weights are scaled by 256 / (256 - p8)
      if (SPLIT && row < Nq) {
#pragma unroll
        for (int c = 0; c < ND32; ++c)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int dcol = c * 32 + 8 * rg + 4 * hi;
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            if (live)
              st = f32x4{oacc[qb][c][4 * rg] * inv, oacc[qb][c][4 * rg + 1] * inv,
                         oacc[qb][c][4 * rg + 2] * inv, oacc[qb][c][4 * rg + 3] * inv};
            *reinterpret_cast<f32x4 *>(p.opart + (pbase + row) * D + dcol) = st;
          }
        if (hi == 0)
          p.lpart[pbase + row] = live ? (mrun[qb] + fast_log2(lt)) * 0.69314718055994531f : -__builtin_inff();
      } else if (!SPLIT && row < Nq) {
#pragma unroll
        for (int c = 0; c < ND32; ++c)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int dcol = c * 32 + 8 * rg + 4 * hi;
            u32x2 st = {0u, 0u};
            if (live) {
              st[0] = T::pack(oacc[qb][c][4 * rg + 0] * inv, oacc[qb][c][4 * rg + 1] * inv);
              st[1] = T::pack(oacc[qb][c][4 * rg + 2] * inv, oacc[qb][c][4 * rg + 3] * inv);
            }
            *reinterpret_cast<u32x2 *>(Oh + (size_t)row * D + dcol) = st;
          }
        if (hi == 0) Lh[row] = live ? (mrun[qb] + fast_log2(lt)) * 0.69314718055994531f : -__builtin_inff();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the split forward's partials: per query row, with L_s the chunks'
// log-sum-exps and O_s their normalised outputs, LSE = log sum_s exp(L_s) and
// O = sum_s exp(L_s - LSE) O_s -- the block-merge rule of the handbook's
// engineering-implementation pseudocode, applied across chunks.  Chunks that see
// no key have L_s = -inf and weight 0; a row with no visible key at all gets
// O = 0, LSE = -inf.  One wave per row, D / 64 output columns per lane.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float *__restrict__ opart,
                                                          const float *__restrict__ lpart,
                                                          uint16_t *__restrict__ o,
                                                          float *__restrict__ lse, int nsplit,
                                                          int Nq, long rows) {
  constexpr int CPL = D / 64;  // columns per lane
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole waves exit together
  const long bh = row / Nq, i = row % Nq;
  const float *ls = lpart + (size_t)bh * nsplit * Nq + i;  // stride Nq between chunks
  // NaN-propagating maximum: a NaN partial makes the row NaN
  float m = -__builtin_inff();
  for (int s = lane; s < nsplit; s += 64) m = __builtin_elementwise_maximum(m, ls[(size_t)s * Nq]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = __builtin_elementwise_maximum(m, __shfl_xor(m, off, 64));
  float acc[CPL] = {};
  float wsum = 0.f;
  if (m != -__builtin_inff()) {
    for (int s = 0; s < nsplit; ++s) {
      const float w = __expf(ls[(size_t)s * Nq] - m);  // 0 for chunks with L_s = -inf
      wsum += w;
      const float *os = opart + (((size_t)bh * nsplit + s) * Nq + i) * D + lane * CPL;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += w * os[c];
    }
  }
  const bool live = wsum != 0.f;  // no visible key: 0; NaN stays NaN
  uint16_t *orow = o + (size_t)row * D + lane * CPL;
  if constexpr (CPL == 2) {
    *reinterpret_cast<uint32_t *>(orow) = live ? T::pack(acc[0] / wsum, acc[1] / wsum) : 0u;
  } else {
    const uint32_t pk = live ? T::pack(acc[0] / wsum, 0.f) : 0u;
    orow[0] = (uint16_t)(pk & 0xFFFFu);
  }
  if (lane == 0) lse[row] = live ? m + __logf(wsum) : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// Decode: one query row per (batch, head) against a long K/V.  Per head this
// is two matrix-vector products (scores = K q, o = V^T p) that read every K
// and V byte once and do 2 FLOP per byte: bound by HBM, not by the matrix
// cores, and an MFMA tile would be 31/32 padding.  So the kernel streams K
// and V through registers with wave-wide 16-byte loads and works on the
// vector ALUs: v_dot2 for the scores, FMAs for the output.
//
// Lane roles: a row of d 16-bit values is LPK = d/8 lanes of 16 bytes, so one
// load covers KPL = 64/LPK consecutive key rows; lane = (key slot g, column
// chunk u).  Each wave takes its own chunk of p.chunk keys with its own online
// softmax (running max in the log2 domain, rescale of the running sum and
// output at every tile) and writes one partial: the chunk's normalised output
// and LSE, merged by fwd_combine_kernel like the split forward's partials.
// p.nsplit = partials per head = 4 x workgroups per head.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(256) void fwd_decode_kernel(FwdParams p) {
  constexpr int RB = D * 2;      // bytes per row
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPL = 64 / LPK;  // key rows per load
  constexpr int NI = 8;          // loads per tensor per tile
  constexpr int TK = NI * KPL;   // keys per tile: 32 (d = 128) or 64 (d = 64)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane / LPK, u = lane % LPK;
  const int wg_per_head = p.nsplit / 4;
  const int bh = blockIdx.x / wg_per_head;
  const int split = (blockIdx.x % wg_per_head) * 4 + w;
  int Lq, Lk;
  seq_lengths(p.seq, bh / p.seq.H, Lq, Lk);
  // the single query sees keys [0, Lk) (causal changes nothing when Nq = 1);
  // a padding row (Lq = 0) sees none
  const int j0 = split * p.chunk;
  const int j1 = Lq > 0 ? min(j0 + p.chunk, Lk) : 0;
  const size_t koff = (size_t)bh * (size_t)p.seq.Nk * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const uint16_t *>(p.k) + koff, (uint32_t)Lk * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const uint16_t *>(p.v) + koff, (uint32_t)Lk * RB);
  const u32x4 qv = gload16(reinterpret_cast<const uint16_t *>(p.q) + (size_t)bh * D + u * 8);
  const float sl2 = p.scale_log2;

  float m = -__builtin_inff(), l = 0.f;  // running max (log2 domain) and this key slot's sum
  float o[8] = {};                       // columns 8u .. 8u + 7, this key slot's keys
  for (int t0 = j0; t0 < j1; t0 += TK) {
    u32x4 kv[NI], vv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t off = (uint32_t)((t0 + i * KPL + g) * RB + u * 16);  // rows past Lk read 0
      kv[i] = bload16(rk, off);
      vv[i] = bload16(rv, off);
    }
    // scores of the tile's keys (key t0 + i KPL + g), log2 domain, masked past j1
    float s[NI];
    float mt = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float dt = T::dot2(kv[i][0], qv[0], 0.f);
      dt = T::dot2(kv[i][1], qv[1], dt);
      dt = T::dot2(kv[i][2], qv[2], dt);
      dt = T::dot2(kv[i][3], qv[3], dt);
      dt = group_sum<LPK>(dt);
      s[i] = t0 + i * KPL + g < j1 ? dt * sl2 : -__builtin_inff();
      mt = __builtin_elementwise_maximum(mt, s[i]);  // NaN-propagating (v_maximum3_f32)
    }
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) mt = __builtin_elementwise_maximum(mt, __shfl_xor(mt, off, 64));
    const float mn = __builtin_elementwise_maximum(m, mt);
    if (mn == -__builtin_inff()) continue;  // wave-uniform: no visible key yet
    const float alpha = fast_exp2(m - mn);  // 0 while m = -inf
    m = mn;
    float ls = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pr = fast_exp2(s[i] - mn);  // masked: exp2(-inf) = 0
      ls += pr;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[2 * c] = __builtin_fmaf(pr, T::lo(vv[i][c]), o[2 * c]);
        o[2 * c + 1] = __builtin_fmaf(pr, T::hi(vv[i][c]), o[2 * c + 1]);
      }
    }
    l = l * alpha + ls;
  }
  // totals over the key slots (lanes with the same column chunk)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] += __shfl_xor(o[c], off, 64);
  }
  const bool live = l != 0.f;  // no visible key: 0; NaN stays NaN
  const size_t prow = (size_t)bh * p.nsplit + split;  // Nq = 1
  if (g == 0) {
    const float inv = live ? 1.f / l : 0.f;
    float *op = p.opart + prow * D + u * 8;
    *reinterpret_cast<f32x4 *>(op) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4 *>(op + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
  }
  if (lane == 0) p.lpart[prow] = live ? (m + fast_log2(l)) * 0.6931471805599453f : -__builtin_inff();
}

// ---------------------------------------------------------------------------
// instantiation table
// ---------------------------------------------------------------------------

template <class T, int D, int QB, bool C>
static hipError_t launch_fwd_t(const FwdParams &p, int grid, hipStream_t st) {
  if (p.drop.p8 != 0)
    hipLaunchKernelGGL((fwd_kernel<T, D, QB, C, true, false>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, QB, C, false, false>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class T, int D, bool C>
static hipError_t launch_split_t(const FwdParams &p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<T, D, 1, C, false, true>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_fwd_split(const FwdParams &p, int dtype, int d, int causal, int grid,
                            hipStream_t st) {
  if (dtype == 1)
    return d == 128 ? (causal ? launch_split_t<BF16, 128, true>(p, grid, st) : launch_split_t<BF16, 128, false>(p, grid, st))
                    : (causal ? launch_split_t<BF16, 64, true>(p, grid, st) : launch_split_t<BF16, 64, false>(p, grid, st));
  return d == 128 ? (causal ? launch_split_t<F16, 128, true>(p, grid, st) : launch_split_t<F16, 128, false>(p, grid, st))
                  : (causal ? launch_split_t<F16, 64, true>(p, grid, st) : launch_split_t<F16, 64, false>(p, grid, st));
}

template <class T, int D>
static hipError_t launch_decode_t(const FwdParams &p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_decode_kernel<T, D>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_fwd_decode(const FwdParams &p, int dtype, int d, int grid, hipStream_t st) {
  if (dtype == 1) return d == 128 ? launch_decode_t<BF16, 128>(p, grid, st) : launch_decode_t<BF16, 64>(p, grid, st);
  return d == 128 ? launch_decode_t<F16, 128>(p, grid, st) : launch_decode_t<F16, 64>(p, grid, st);
}

template <class T, int D>
static hipError_t launch_combine_t(const FwdParams &p, long rows, hipStream_t st) {
  const int grid = (int)((rows + 3) / 4);
  hipLaunchKernelGGL((fwd_combine_kernel<T, D>), dim3(grid), dim3(256), 0, st, p.opart, p.lpart,
                     reinterpret_cast<uint16_t *>(p.o), p.lse, p.nsplit, p.seq.Nq, rows);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const FwdParams &p, int dtype, int d, long rows, hipStream_t st) {
  if (dtype == 1) return d == 128 ? launch_combine_t<BF16, 128>(p, rows, st) : launch_combine_t<BF16, 64>(p, rows, st);
  return d == 128 ? launch_combine_t<F16, 128>(p, rows, st) : launch_combine_t<F16, 64>(p, rows, st);
}

hipError_t launch_fwd(const FwdParams &p, int dtype, int d, int causal, int qb, int grid,
                      hipStream_t st) {
#define FA_FWD_CASE(TT, DD, QQ)                                                       \
  if (d == DD && qb == QQ) {                                                          \
    return causal ? launch_fwd_t<TT, DD, QQ, true>(p, grid, st)                       \
                  : launch_fwd_t<TT, DD, QQ, false>(p, grid, st);                     \
  }
  if (dtype == 1) {
    FA_FWD_CASE(BF16, 128, 1)
    FA_FWD_CASE(BF16, 64, 1)
#if FWD_QB_D64 != 1
    FA_FWD_CASE(BF16, 64, FWD_QB_D64)
#endif
  } else {
    FA_FWD_CASE(F16, 128, 1)
    FA_FWD_CASE(F16, 64, 1)
#if FWD_QB_D64 != 1
    FA_FWD_CASE(F16, 64, FWD_QB_D64)
#endif
  }
#undef FA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
