// Threshold selection of the LoSA construction step on gfx950.
//
// One wavefront per query block (row of the mass map).  The row's nkb
// masses become 64-bit keys (fp32 bit pattern << 32 | ~block index): masses
// are >= +0, so the bit pattern orders like the value, and the complemented
// index breaks ties toward the smaller block.  The keys are sorted
// descending in registers by a bitonic network (E = pow2(nkb)/64 keys per
// lane; exchanges across lanes via cross-lane shuffles), then a float64
// prefix sum in sorted order finds the first position where the running mass
// reaches the threshold.  Float64 sums of float32 masses >= 2^-30 are exact
// below 1 under any association, so the parallel scan decides exactly like
// a sequential accumulation.  The threshold is one value for every row, or
// (per-row variant) taus[row / rows_per_tau] read from device memory.
#include "losa_device.h"
#include "losa_launch.h"

namespace losa {

// The value of v held by lane l ^ lj.  Distances 1 and 2 are quad
// permutations, 4 a mirror of each 8-lane half row (lane i reads i ^ 7)
// followed by a quad reversal (i ^ 3), and 8 a rotation of each 16-lane row
// by 8 (the same as xor 8 there): DPP moves, ordinary VALU work with no
// wait.  Distances 16 and 32 cross rows and go through ds_bpermute.
__device__ __forceinline__ unsigned long long lane_xor64(unsigned long long v, int lj) {
  const int lo = (int)(unsigned)v, hi = (int)(unsigned)(v >> 32);
  int rlo, rhi;
  if (lj == 1) {
    rlo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
    rhi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, true);
  } else if (lj == 2) {
    rlo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
    rhi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, true);
  } else if (lj == 4) {
    rlo = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, true), 0x1B,
                                   0xF, 0xF, true);  // row_half_mirror, quad_perm [3,2,1,0]
    rhi = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, true), 0x1B,
                                   0xF, 0xF, true);
  } else if (lj == 8) {
    rlo = __builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, true);  // row_ror:8
    rhi = __builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, true);
  } else {
    return __shfl_xor(v, lj, 64);
  }
  return ((unsigned long long)(unsigned)rhi << 32) | (unsigned)rlo;
}

template <int E>
__global__ void __launch_bounds__(256) select_kernel(const float* __restrict__ mass, int rows,
                                                     int nkb, double tau,
                                                     const double* __restrict__ taus,
                                                     int rows_per_tau,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ count) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // no barriers below: whole waves leave together
  if (taus != nullptr) tau = taus[row / rows_per_tau];
  const float* __restrict__ m = mass + (size_t)row * nkb;

  unsigned long long key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int e = lane * E + r;
    unsigned long long kv = 0ull;  // padding sorts after every real key
    if (e < nkb) {
      unsigned bits = __float_as_uint(m[e]);
      if (bits >> 31) bits = 0u;  // negative masses are treated as zero
      kv = ((unsigned long long)bits << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)e);
    }
    key[r] = kv;
  }

  // bitonic sort, descending: in a k-block whose (e & k) == 0 the lower
  // position keeps the larger key.  Each compare-exchange is one 64-bit
  // compare whose outcome is flipped by the block's direction, then one
  // select per word.  For k < E the direction depends only on r, for
  // k >= E only on the lane (e = lane * E + r).
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
    const bool lane_desc = ((lane * E) & k) == 0;  // the direction when k >= E
#pragma unroll
    for (int j = k >> 1; j >= 1; j >>= 1) {
      if (j >= E) {
        const int lj = j / E;
        const bool lower = (lane & lj) == 0;
        const bool take_max = (lower == lane_desc);  // here k > j >= E
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const unsigned long long other = lane_xor64(key[r], lj);
          const bool keep = (key[r] > other) == take_max;
          key[r] = keep ? key[r] : other;
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if ((r & j) == 0) {
            const int r2 = r | j;
            const bool desc = k < E ? ((r & k) == 0) : lane_desc;
            const unsigned long long a = key[r], b = key[r2];
            const bool swap = (a < b) == desc;
            key[r] = swap ? b : a;
            key[r2] = swap ? a : b;
          }
        }
      }
    }
  }

  // float64 inclusive prefix of the sorted masses
  double pre[E];
  double run = 0.0;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    run += (double)__uint_as_float((unsigned)(key[r] >> 32));
    pre[r] = run;
  }
  double incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;

  int first = nkb;  // first sorted position whose prefix reaches tau
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int e = lane * E + r;
    if (e < nkb && excl + pre[r] >= tau) first = min(first, e);
  }
  first = wave_min(first);
  const int cnt = (tau >= 1.0 || first >= nkb) ? nkb : first + 1;

  int32_t* __restrict__ out = idx + (size_t)row * nkb;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int e = lane * E + r;
    if (e < cnt) out[e] = (int32_t)(0xFFFFFFFFu - (unsigned)(key[r] & 0xFFFFFFFFull));
  }
  if (lane == 0) count[row] = cnt;
}

hipError_t launch_select(int32_t rows, int32_t nkb, const float* mass, double tau,
                         const double* taus, int32_t rows_per_tau, int32_t* idx, int32_t* count,
                         hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (nkb <= 64) {
    hipLaunchKernelGGL(select_kernel<1>, grid, block, 0, stream, mass, rows, nkb, tau, taus,
                       rows_per_tau, idx, count);
  } else if (nkb <= 128) {
    hipLaunchKernelGGL(select_kernel<2>, grid, block, 0, stream, mass, rows, nkb, tau, taus,
                       rows_per_tau, idx, count);
  } else if (nkb <= 256) {
    hipLaunchKernelGGL(select_kernel<4>, grid, block, 0, stream, mass, rows, nkb, tau, taus,
                       rows_per_tau, idx, count);
  } else if (nkb <= 512) {
    hipLaunchKernelGGL(select_kernel<8>, grid, block, 0, stream, mass, rows, nkb, tau, taus,
                       rows_per_tau, idx, count);
  } else if (nkb <= 1024) {
    hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, stream, mass, rows, nkb, tau, taus,
                       rows_per_tau, idx, count);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace losa
