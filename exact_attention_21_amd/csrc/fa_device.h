// Device-side building blocks for the gfx950 attention kernels: vector types,
// the 32x32x16 MFMA for fp16/bf16 inputs, fp32 -> 16-bit packing, LDS access
// (plain and transposing reads) and the cross-half-wave exchange.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16} register layout (wave64), verified on the
// device by a lane-layout probe:
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + j], j = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + j][l % 32], j = 0..7
//   C (32 x 32): lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// The contraction index may be relabelled freely as long as A and B agree.
//
// ds_read_b64_tr_b16 (per 16-lane group): source lane s supplies the address of
// four consecutive 16-bit values; destination lane i receives element (i % 4)
// of source lanes 4t + i / 4 for t = 0..3.  If source lane s points at
// row r0 + s / 4, columns c0 + 4 (s % 4) .. +3 of a row-major matrix, lane i
// receives rows r0..r0+3 of column c0 + i: a transposed 4 x 16 block.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct BF16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 values -> packed pair, round to nearest even (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
  static __device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
  // c + a.lo * b.lo + a.hi * b.hi (v_dot2_f32_bf16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Two fp32 values -> packed pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  }
  static __device__ __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(f16x2, u)[0];
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(f16x2, u)[1];
  }
  // c + a.lo * b.lo + a.hi * b.hi (v_dot2_f32_f16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
};

// Value of lane l ^ 32 (the other half-wave), via v_permlane32_swap.
__device__ __forceinline__ float xhalf(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // lanes 0..31: r[1] holds lane l+32's value; lanes 32..63: r[0] holds lane l-32's.
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float max_xhalf(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_xhalf(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over each group of N consecutive lanes (N = 8 or 16), left in every lane
// of the group: DPP swaps with lane ^ 1 and lane ^ 2, then the mirror images
// within 8 and within 16 lanes.  Both lanes of every exchange add the same two
// values, so the group's lanes end with bitwise-equal sums.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, true));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N == 16) x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

// Workgroup -> (head, tile rank) for a 1-D grid of heads x ntiles workgroups.
// With xcd_grouped (heads a multiple of 8) workgroup bid runs on XCD bid % 8
// and only heads bh with bh % 8 == bid % 8 go there.  The heads of an XCD are
// taken in groups of `group`, and its last `tail` heads form one group of
// their own; within a group every head's rank-0 tile comes first, then every
// rank-1 tile, and so on.  group = 1: a head's tiles are consecutive, so they
// run together and share its K/V in L2; larger groups interleave more heads
// (more L2 traffic) but, with rank 0 the longest tile of a causal mask, end
// the grid on shorter tiles; the tail group evens out the end of the grid.
__host__ __device__ __forceinline__ void grid_tile(int bid, int heads, int ntiles, bool xcd_grouped,
                                                   int group, int tail, int &bh, int &rank) {
  const int lanes = xcd_grouped ? 8 : 1;                 // heads interleaved across XCDs
  const int x = xcd_grouped ? (bid & 7) : 0, kk = xcd_grouped ? (bid >> 3) : bid;
  const int hpx = heads / lanes;                         // heads of this XCD (or of the grid)
  const int nt = min(max(tail, 0), hpx), nrest = hpx - nt;
  int h;
  if (kk < nrest * ntiles) {
    const int gi = kk / (group * ntiles), idx = kk % (group * ntiles);
    const int gsz = min(group, nrest - gi * group);      // the last group may be smaller
    rank = idx / gsz;
    h = gi * group + idx % gsz;
  } else {
    const int idx = kk - nrest * ntiles;
    rank = idx / nt;
    h = nrest + idx % nt;
  }
  bh = x + lanes * h;
}

__device__ __forceinline__ u32x4 lds_read16(const char *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void lds_write16(char *p, u32x4 v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}

// Transposing LDS read of four 16-bit values (see the layout note above).
__device__ __forceinline__ u32x2 lds_read_tr4(const char *p) {
  s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
  return __builtin_bit_cast(u32x2, t);
}

__device__ __forceinline__ u32x4 gload16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Raw buffer resource over `bytes` bytes at `base`; loads past the end return 0
// (hardware range check), so ragged tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// A wave-uniform pointer moved to scalar registers (so that a buffer resource
// built from it needs no per-lane handling).
__device__ __forceinline__ const char *uniform_ptr(const char *ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
}

// Buffer resource of one tile of a tensor whose first `valid` bytes at `base`
// hold data: it starts at byte tb and ends where the valid bytes end (rows
// past it read as zeros), so the per-lane offsets of the tile's loads stay
// loop-invariant; ok = false gives an empty record (every load reads zeros).
// The arguments are wave-uniform; unsigned, so that a tensor may span up to
// 2^32 - 1 bytes.  The record size valid - tb, or 0 where the unsigned
// subtraction borrows (tb >= valid), takes two scalar instructions; written in
// C the compiler takes the saturating subtraction to the vector ALU (a move, a
// clamped subtraction, a select and a readfirstlane per tile).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *base, uint32_t tb, uint32_t valid, bool ok) {
  const uint32_t t = __builtin_amdgcn_readfirstlane(ok ? tb : 0u);
  const uint32_t v = __builtin_amdgcn_readfirstlane(ok ? valid : 0u);
  uint32_t n;
  asm("s_sub_u32 %0, %1, %2\n\ts_cselect_b32 %0, 0, %0" : "=&s"(n) : "s"(v), "s"(t) : "scc");
  return make_rsrc(uniform_ptr(base + t), n);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Direct global -> LDS load of 16 bytes per lane: lane i of the wave writes
// lds_block + 16 i (the block address must be wave-uniform).  Offsets past the
// resource's end write zeros.  Completion is tracked by vmcnt only.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds_block, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_block, 16, byte_off, 0, 0, 0);
}

// s_waitcnt with only vmcnt constrained (expcnt, lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without the memory fences of __syncthreads (which would
// also drain every outstanding global load).  It first waits for this wave's
// own LDS reads: the compiler may sink the arithmetic that consumes a read
// below the barrier, and the read must not still be in flight when another
// wave passes the barrier and starts overwriting that LDS.  The memory clobber
// keeps the compiler from moving LDS accesses across it.  Callers wait (vmcnt)
// for the buffer->LDS loads that must have landed before calling it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Output tiles leave through LDS.  A wave's 32 x D tile of 16-bit values
// comes out of a transposed 32x32 accumulator with lane l holding row l % 32,
// columns c * 32 + 8 rg + 4 (l / 32) .. + 3 as two packed pairs per (c, rg).
// Stored directly, every store instruction would write 16 bytes into each of
// 32 rows; instead each pair goes to `stage` (32 * D * 2 bytes of LDS that
// only this wave uses, 16-byte chunks XOR-swizzled by row: stage_put), and
// the rows come back one 16-byte piece per lane, so that each store writes
// whole rows (stage_store_rows).
template <int D>
__device__ __forceinline__ void stage_put(char *stage, int c, int rg, u32x2 v, int lane) {
  constexpr int RB = D * 2, CPR = RB / 16;  // row bytes, 16-byte chunks per row
  const int l32 = lane & 31, hi = lane >> 5;
  *reinterpret_cast<u32x2 *>(stage + l32 * RB + (((4 * c + rg) ^ (l32 & (CPR - 1))) << 4) + 8 * hi) = v;
}
// Rows row0 .. row0 + 31 of the row-major [rows][D] array dst, those below
// nrows, from the staged tile; the stage may be reused after it returns.
template <int D>
__device__ __forceinline__ void stage_store_rows(const char *stage, uint16_t *dst, int row0, int nrows, int lane) {
  constexpr int RB = D * 2, CPR = RB / 16, RPI = 64 / CPR;  // rows per store
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is in LDS before it is read back
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CPR, ch = lane % CPR;
    const u32x4 x = lds_read16(stage + r * RB + ((ch ^ (r & (CPR - 1))) << 4));
    if (row0 + r < nrows) *reinterpret_cast<u32x4 *>(dst + (size_t)(row0 + r) * D + ch * 8) = x;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the stage is written again
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32 (base 2)

// ---- dropout mask ------------------------------------------------------------
// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw
// ("Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds, each
// multiplying counter words 0 and 2 by two fixed odd constants into 64-bit
// products whose halves are permuted and xored with the other counter words and
// the key; the key advances by a Weyl increment between rounds.  The key is
// uniform across the wave, so its schedule stays in scalar registers.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // 64-bit products: one v_mad_u64_u32 each instead of a mul_lo / mul_hi pair
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c = u32x4{hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0};
  }
  return c;
}

// 4x4 transpose of words across each group of four consecutive lanes: lane t
// returns w[s] = (lane s of its group).x[t].  Two butterfly stages: exchange
// with lane t ^ 1 the registers whose index differs from t in bit 0, then with
// lane t ^ 2 those differing in bit 1 (DPP quad permutations).
__device__ __forceinline__ u32x4 quad_transpose(u32x4 x) {
  const int t = threadIdx.x & 3;
  auto swap1 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true); };  // [1,0,3,2]
  auto swap2 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true); };  // [2,3,0,1]
  const bool odd = t & 1, high = t & 2;
  const uint32_t p0 = swap1(x[0]), p1 = swap1(x[1]), p2 = swap1(x[2]), p3 = swap1(x[3]);
  const u32x4 y = {odd ? p1 : x[0], odd ? x[1] : p0, odd ? p3 : x[2], odd ? x[3] : p2};
  const uint32_t q0 = swap2(y[0]), q1 = swap2(y[1]), q2 = swap2(y[2]), q3 = swap2(y[3]);
  return u32x4{high ? q2 : y[0], high ? q3 : y[1], high ? y[2] : q0, high ? y[3] : q1};
}

// 4x4 transpose of bytes inside a lane: y[t] byte s = x[s] byte t.
__device__ __forceinline__ u32x4 byte_transpose(u32x4 x) {
  // (x0 b_i, x1 b_i, x0 b_i+1, x1 b_i+1) for i = 0, 2, and the same for x2, x3
  const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  return u32x4{__builtin_amdgcn_perm(lo23, lo01, 0x05040100u), __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
               __builtin_amdgcn_perm(hi23, hi01, 0x05040100u), __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
}

// Dropout bytes of the 16 (query, key) pairs an MFMA accumulator lane holds:
// byte b of word a belongs to register r = 4a + b.  A pair (i, j) of head bh is
// kept iff byte j % 4 of word i % 4 of Philox(counter = (j / 4, i / 4, bh,
// offset), key) >= p8 (see kept()).
// Query-major lanes (one query i, keys j0 + 8a + 4hi + b): the lane computes the
// block of key group j0/4 + 2t + hi (t = i % 4, quad member), and the quad
// transpose hands every lane word i % 4 of the four blocks it needs.
__device__ __forceinline__ u32x4 keep_bytes_query_major(int i, int j0, int hi, uint32_t bh,
                                                        uint32_t offset, uint32_t k0, uint32_t k1) {
  const int t = i & 3;
  const u32x4 r = philox4x32_10(u32x4{(uint32_t)(j0 / 4 + 2 * t + hi), (uint32_t)(i / 4), bh, offset}, k0, k1);
  return quad_transpose(r);
}
// Key-major lanes (one key j, queries i0 + 8a + 4hi + b): the lane computes the
// block of query group i0/4 + 2t + hi (t = j % 4), gathers byte t' of its four
// words for each quad member t', and the quad transpose hands lane t the bytes
// of key offset t for the four query groups.
__device__ __forceinline__ u32x4 keep_bytes_key_major(int j, int i0, int hi, uint32_t bh,
                                                      uint32_t offset, uint32_t k0, uint32_t k1) {
  const int t = j & 3;
  const u32x4 r = philox4x32_10(u32x4{(uint32_t)(j / 4), (uint32_t)(i0 / 4 + 2 * t + hi), bh, offset}, k0, k1);
  return quad_transpose(byte_transpose(r));
}
// Whether register r's pair is kept (a byte compare, SDWA on gfx950).
__device__ __forceinline__ bool kept(const u32x4 &w, int r, uint32_t p8) {
  return ((w[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= p8;
}

}  // namespace fa
