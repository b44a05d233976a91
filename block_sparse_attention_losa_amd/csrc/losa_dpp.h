// Exchanges inside a 16-lane DPP row (gfx950): VALU moves, no LDS round trip.
#pragma once

#include <hip/hip_runtime.h>

namespace losa {

// The 32-bit value held by lane l ^ LJ, LJ in {1, 2, 4, 8}, all within a
// 16-lane row: distances 1 and 2 are quad permutations, 4 a mirror of each
// 8-lane half row (lane i reads i ^ 7) followed by a quad reversal (i ^ 3),
// 8 a rotation of the row by 8.
template <int LJ>
__device__ __forceinline__ int row_xor(int v) {
  static_assert(LJ == 1 || LJ == 2 || LJ == 4 || LJ == 8, "lane distance inside a DPP row");
  if constexpr (LJ == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  if constexpr (LJ == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  if constexpr (LJ == 4)
    return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true), 0x1B,
                                    0xF, 0xF, true);
  return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);
}

template <int LJ>
__device__ __forceinline__ float row_xor(float v) {
  return __int_as_float(row_xor<LJ>(__float_as_int(v)));
}

template <int LJ>
__device__ __forceinline__ double row_xor(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = row_xor<LJ>((int)(unsigned)u), hi = row_xor<LJ>((int)(unsigned)(u >> 32));
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Sum over the 16 lanes of the row, the same bits in every lane (a
// butterfly: each lane adds the same pairs, and float addition commutes).
__device__ __forceinline__ float row_sum16(float x) {
  x += row_xor<1>(x);
  x += row_xor<2>(x);
  x += row_xor<4>(x);
  return x + row_xor<8>(x);
}

}  // namespace losa
