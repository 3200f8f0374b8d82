// Shared by the two backward passes (fa_bwd.hip: the row statistics and the
// dQ pass; fa_bwd_dkdv.h: the dK/dV pass): the LDS swizzles of the streamed
// tiles and the occupancy targets.
#pragma once

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

// XOR swizzles of the 16-byte chunk index within a 256-byte (d = 128) or
// 128-byte (d = 64) tile row.  FRAG: conflict-free for 16-byte fragment reads
// of 32 consecutive rows; BOTH: also conflict-free for the transposing reads
// of 4 consecutive rows.
template <int D>
__device__ __forceinline__ int swz_frag(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__host__ __device__ constexpr int swz_both(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row & 3) << 1) ^ ((row >> 2) & 3)) & 7);
}
// Both swizzles repeat every 16 rows, so a fragment address precomputed for
// rows r .. r + 15 serves rows r + 16 .. r + 31 with a constant offset.
template <int D>
constexpr bool swz_period16() {
  for (int r = 0; r < 16; ++r)
    if (swz_both<D>(r + 16) != swz_both<D>(r) || ((r + 16) & 15) != (r & 15)) return false;
  return true;
}
static_assert(swz_period16<64>() && swz_period16<128>(), "swizzles must repeat every 16 rows");

}  // namespace

// waves per SIMD of the two passes (occupancy targets; d = 64 needs fewer registers)
#define BWD_DQ_OCC(D, DROP) ((D) == 64 && !(DROP) ? BWD_DQ_WAVES_D64 : BWD_DQ_WAVES_PER_SIMD)
#define BWD_DKDV_OCC(D, DROP) ((D) == 64 && !(DROP) ? BWD_DKDV_WAVES_D64 : BWD_DKDV_WAVES_PER_SIMD)

}  // namespace fa
