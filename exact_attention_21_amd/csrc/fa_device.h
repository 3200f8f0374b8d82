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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32 (base 2)

}  // namespace fa
