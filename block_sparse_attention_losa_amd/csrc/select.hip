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
  // position keeps the larger key
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j >= 1; j >>= 1) {
      if (j >= E) {
        const int lj = j / E;
        const bool lower = (lane & lj) == 0;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const unsigned long long other = __shfl_xor(key[r], lj, 64);
          const int e = lane * E + r;
          const bool desc = (e & k) == 0;
          const bool take_max = (lower == desc);
          const unsigned long long hi = key[r] > other ? key[r] : other;
          const unsigned long long lo = key[r] > other ? other : key[r];
          key[r] = take_max ? hi : lo;
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if ((r & j) == 0) {
            const int r2 = r | j;
            const int e = lane * E + r;
            const bool desc = (e & k) == 0;
            const unsigned long long a = key[r], b = key[r2];
            const unsigned long long hi = a > b ? a : b;
            const unsigned long long lo = a > b ? b : a;
            key[r] = desc ? hi : lo;
            key[r2] = desc ? lo : hi;
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
