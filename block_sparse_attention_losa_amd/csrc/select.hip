// Threshold selection of the LoSA construction step on gfx950.
//
// Per row of the mass map: order the key blocks by descending mass (ties
// toward the smaller block index), accumulate the masses in that order in
// float64, and keep the shortest prefix whose sum reaches the threshold.
//
// A row's nkb masses become 64-bit keys (fp32 bit pattern << 30 | 2^30-1-J):
// masses are >= +0, so the pattern orders like the value, and the
// complemented index breaks ties toward the smaller block.  Read as IEEE
// doubles these keys are finite and non-negative (the top three bits are
// zero, so the exponent field is at most 0x1FF) and order exactly like the
// integers; a mass of 0 gives a denormal double, which these kernels keep
// (float64 denormals are enabled).  A compare-exchange inside a lane is then
// one v_max_f64 and one v_min_f64 (float64 max and min issue at full rate,
// float64 compares far slower).  The keys are sorted by a bitonic network
// over P = pow2(nkb) positions held by L lanes, E = P/L per lane
// (position = lane * E + register), with E = 16 and L = P/16 for long rows
// and L = 16 for short ones (measured fastest: enough exchanges stay inside
// a lane while registers stay below ~100, so several waves share a SIMD).
// Exchanges at distances below E stay in a lane, lane distances 1-8 are DPP
// moves inside a 16-lane row and 16, 32 ds_bpermute.  Where the direction of
// a bitonic block depends on the lane, the lane's keys are negated for that
// stage (min(a, b) = -max(-a, -b)), so every exchange in the stage keeps the
// larger value at the lower position.  A float64 prefix sum in sorted order
// then finds the first position where the running mass reaches the
// threshold.  Float64 sums of float32 masses >= 2^-30 are exact below 1
// under any association, so the parallel scan decides exactly like a
// sequential accumulation.  The threshold is one value for every row, or
// (per-row variant) taus[row / rows_per_tau].
#include "losa_device.h"
#include "losa_launch.h"

namespace losa {

namespace {

// The value held by lane ^ LJ: DPP inside a 16-lane row, ds_bpermute across.
template <int LJ>
__device__ __forceinline__ double lane_xor(double v) {
  if constexpr (LJ <= 8) {
    return row_xor<LJ>(v);
  } else {
    return __shfl_xor(v, LJ, 64);
  }
}
template <int LJ>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (LJ <= 8) {
    return row_xor<LJ>(v);
  } else {
    return __shfl_xor(v, LJ, 64);
  }
}

// A DPP move of a double (both halves), 0 in lanes the control leaves
// without a source or whose row is not in ROWMASK.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROWMASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROWMASK, 0xF,
                                             false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Inclusive prefix sum over the L lanes of a mass-map row, all in DPP: a
// Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8), then for
// L >= 32 the last lane of rows 0 and 2 added to rows 1 and 3 (row_bcast:15)
// and for L = 64 lane 31 added to rows 2 and 3 (row_bcast:31).
template <int L>
__device__ __forceinline__ double row_scan(double x) {
  x += dpp_f64<0x111>(x);
  x += dpp_f64<0x112>(x);
  x += dpp_f64<0x114>(x);
  x += dpp_f64<0x118>(x);
  if constexpr (L >= 32) x += dpp_f64<0x142, 0xA>(x);
  if constexpr (L == 64) x += dpp_f64<0x143, 0xC>(x);
  return x;
}

// Minimum over the L lanes of a mass-map row.
template <int L, int LJ = 1>
__device__ __forceinline__ int row_min(int x) {
  if constexpr (LJ < L) {
    return row_min<L, 2 * LJ>(min(x, lane_xor<LJ>(x)));
  } else {
    return x;
  }
}

// Keys are built from masses >= 0 (negative ones count as 0) and block
// indices < 2^30; 0.0 pads positions past nkb and sorts after every key.
__device__ __forceinline__ double make_key(float m, int j) {
  const int bits = max((int)__float_as_uint(m), 0);
  const unsigned long long k =
      ((unsigned long long)(unsigned)bits << 30) | (unsigned long long)(0x3FFFFFFFu - (unsigned)j);
  return __longlong_as_double((long long)k);
}
__device__ __forceinline__ float key_mass(double k) {
  return __uint_as_float((unsigned)((unsigned long long)__double_as_longlong(k) >> 30));
}
__device__ __forceinline__ int key_block(double k) {
  return (int)(0x3FFFFFFFu - ((unsigned)__double_as_longlong(k) & 0x3FFFFFFFu));
}

// +1 in a lane whose `bit` is clear, -1 where it is set.
__device__ __forceinline__ double lane_sign(int l, int bit) { return (l & bit) == 0 ? 1.0 : -1.0; }

// Cross-lane steps at lane distances LJ, LJ/2, ..., 1 of a folded stage (the
// larger key goes to the lower position).  During a step the lane holds
// g = t * f, f its folded key and t = +1 in the lower lane of each pair, -1
// in the upper one, so the partner holds -t * f'; then max(g, -g') is t times
// the key the lane keeps (max(f, f') below, min(f, f') above): two v_max_f64
// and no compare (float64 compares issue far slower than max and min).
// Entering a step the keys carry the step's t; leaving it they are switched
// to the next step's t, and after the last one back to plain folded keys.
template <int E, int LJ>
__device__ __forceinline__ void cross_steps(double (&key)[E], int l) {
  if constexpr (LJ >= 1) {
#pragma unroll
    for (int r = 0; r < E; ++r) key[r] = fmax(key[r], -lane_xor<LJ>(key[r]));
    const double flip = lane_sign(l, LJ) * (LJ > 1 ? lane_sign(l, LJ / 2) : 1.0);
#pragma unroll
    for (int r = 0; r < E; ++r) key[r] *= flip;
    cross_steps<E, LJ / 2>(key, l);
  }
}

// The in-lane steps J, J/2, ..., 1 of stage K: registers r and r | J.  For
// K < E the block's direction depends on r; from K = E on the keys are
// folded and every exchange keeps the larger key at the lower position.
template <int E, int K, int J>
__device__ __forceinline__ void inlane_steps(double (&key)[E]) {
  if constexpr (J >= 1) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      if ((r & J) == 0) {
        const int r2 = r | J;
        const bool desc = K >= E || (r & K) == 0;
        const double hi = fmax(key[r], key[r2]), lo = fmin(key[r], key[r2]);
        key[r] = desc ? hi : lo;
        key[r2] = desc ? lo : hi;
      }
    }
    inlane_steps<E, K, J / 2>(key);
  }
}

// Bitonic stages K, 2K, ..., L*E over positions e = l * E + r (descending
// overall).  In stage K the block containing e runs descending when
// (e & K) == 0: for K < E that depends on r only; for K >= E on the lane
// only, and there each lane's keys are multiplied by dir = +-1 for the
// stage (fold holds the previous stage's dir).
template <int E, int L, int K>
__device__ __forceinline__ void stages(double (&key)[E], int l, double fold) {
  if constexpr (K <= L * E) {
    if constexpr (K >= E) {
      const double dir = ((l * E) & K) == 0 ? 1.0 : -1.0;
      double flip = dir * fold;
      if constexpr (K > E) flip *= lane_sign(l, K / (2 * E));  // the first cross step's t
#pragma unroll
      for (int r = 0; r < E; ++r) key[r] *= flip;
      fold = dir;
    }
    if constexpr (K > E) cross_steps<E, K / (2 * E)>(key, l);
    inlane_steps<E, K, (K > E ? E : K) / 2>(key);
    stages<E, L, 2 * K>(key, l, fold);
  }
}

}  // namespace

template <int E, int L>
__global__ void __launch_bounds__(64) select_kernel(const float* __restrict__ mass, int rows,
                                                    int nkb, double tau,
                                                    const double* __restrict__ taus,
                                                    int rows_per_tau,
                                                    int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ count) {
  constexpr int kRowsPerWave = 64 / L;
  constexpr int kPad = E >= 4 ? 4 : 0;  // LDS words after each lane's run (bank spread)
  constexpr int kRowWords = L * (E + kPad);
  __shared__ int32_t stage[kRowsPerWave * kRowWords];

  const int lane = threadIdx.x;
  const int sub = lane / L, l = lane % L;
  const int row = blockIdx.x * kRowsPerWave + sub;
  const bool live = row < rows;
  const float* __restrict__ m = mass + (size_t)(live ? row : 0) * nkb;

  // register r of lane l holds block r * L + l (coalesced reads); where a
  // key starts does not matter, it carries its own block index
  double key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int j = r * L + l;
    key[r] = (live && j < nkb) ? make_key(m[j], j) : 0.0;
  }

  // bitonic sort, descending
  stages<E, L, 2>(key, l, 1.0);
  // the last stage (K = P) runs descending everywhere: the keys end unfolded

  if (live && taus != nullptr) tau = taus[row / rows_per_tau];
  // prefixes are sums of masses >= +0, where doubles order like their bit
  // patterns: compare those (a threshold <= 0 is reached at once, NaN never)
  const unsigned long long tau_bits =
      tau > 0.0 ? (unsigned long long)__double_as_longlong(tau) : (tau <= 0.0 ? 0ull : ~0ull);

  // float64 prefix of the sorted masses: the lane's sum, an inclusive scan
  // over the row's L lanes, then each position's prefix as the previous
  // lanes' total plus the lane's running sum
  double lane_total = 0.0;
#pragma unroll
  for (int r = 0; r < E; ++r)
    if (l * E + r < nkb) lane_total += (double)key_mass(key[r]);
  const double incl = row_scan<L>(lane_total);
  // the previous lane's prefix: row_shr:1 inside a 16-lane row, wave_shr:1
  // across rows (which hands lane 0 of the next mass-map row a value too)
  double excl = L == 16 ? dpp_f64<0x111>(incl) : dpp_f64<0x138>(incl);
  if (l == 0) excl = 0.0;

  int first = nkb;  // first sorted position whose prefix reaches tau
  double run = 0.0;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int e = l * E + r;
    if (e < nkb) {
      run += (double)key_mass(key[r]);
      if ((unsigned long long)__double_as_longlong(excl + run) >= tau_bits) first = min(first, e);
    }
  }
  first = row_min<L>(first);
  const int cnt = (tau >= 1.0 || first >= nkb) ? nkb : first + 1;

  // kept indices in sorted order, through LDS so that the global stores of
  // a row cover L consecutive entries each
  int32_t* st = stage + sub * kRowWords + l * (E + kPad);
#pragma unroll
  for (int r = 0; r < E; ++r) st[r] = key_block(key[r]);
  __syncthreads();
  if (live) {
    int32_t* __restrict__ out = idx + (size_t)row * nkb;
    const int32_t* rs = stage + sub * kRowWords;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int e = r * L + l;
      if (e < cnt) out[e] = rs[(e / E) * (E + kPad) + (e % E)];
    }
    if (l == 0) count[row] = cnt;
  }
}

hipError_t launch_select(int32_t rows, int32_t nkb, const float* mass, double tau,
                         const double* taus, int32_t rows_per_tau, int32_t* idx, int32_t* count,
                         hipStream_t stream) {
  // P = pow2(nkb) positions: L = max(16, P / 16) lanes per row, E = P / L
#define LOSA_SELECT(P)                                                                         \
  do {                                                                                         \
    constexpr int L = (P) / 16 > 16 ? (P) / 16 : 16;                                           \
    constexpr int E = (P) / L;                                                                 \
    const dim3 grid((unsigned)((rows + 64 / L - 1) / (64 / L))), block(64);                    \
    hipLaunchKernelGGL((select_kernel<E, L>), grid, block, 0, stream, mass, rows, nkb, tau,    \
                       taus, rows_per_tau, idx, count);                                        \
  } while (0)
  if (nkb <= 16) {
    LOSA_SELECT(16);
  } else if (nkb <= 32) {
    LOSA_SELECT(32);
  } else if (nkb <= 64) {
    LOSA_SELECT(64);
  } else if (nkb <= 128) {
    LOSA_SELECT(128);
  } else if (nkb <= 256) {
    LOSA_SELECT(256);
  } else if (nkb <= 512) {
    LOSA_SELECT(512);
  } else if (nkb <= 1024) {
    LOSA_SELECT(1024);
  } else {
    return hipErrorInvalidValue;
  }
#undef LOSA_SELECT
  return hipGetLastError();
}

}  // namespace losa
