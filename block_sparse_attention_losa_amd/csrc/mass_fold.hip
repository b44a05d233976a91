// Mass map from the per-row block sums left by the dense+mass attention pass.
//
// For row i of query block I and key block J the pass stores
//   rowsum[J][i] = log2( sum_{j in J} exp2(c2 s_ij - m_J) ) + (m_J - m0_i)
// and, after its last tile,
//   rowref[i]    = log2( sum_j exp2(c2 s_ij - m_N) ) + (m_N - m0_i),
// where m_J, m_N are the running references in use at those times and m0_i
// the one of the row's first key block (all in log2 units, c2 = c log2 e).
// Then exp2(rowsum[J][i] - rowref[i]) = sum_{j in J} exp(s_ij - lse_i), the
// row's share of the block, and
//   M[I, J] = (1/|I|) sum_{i in I} exp2(rowsum[J][i] - rowref[i])
// is the block mass (mlsanity.com paper index, "Abstract (arXiv)": exact
// block attention masses; ubos.tech blog, "How It Works in Practice",
// Phase 1).
//
// HBM-bound: every stored value is read once (4 bytes per row and key
// block) and one fp32 mass is written per (query block, key block).
#include "losa_device.h"
#include "losa_launch.h"

namespace losa {

// One workgroup per (batch*head, query block I).  Lane l owns rows l (and
// l + 64 for 128-row blocks) of I; a wave takes four key blocks at a time,
// reads each one's rows with one coalesced 256-byte load per 64 rows, and
// sums over the rows with a butterfly (a fixed order, so the result is
// deterministic).
__global__ void __launch_bounds__(256) mass_fold_kernel(const float* __restrict__ rowsum,
                                                        const float* __restrict__ rowref,
                                                        float* __restrict__ mass, int n, int nb,
                                                        int block) {
  constexpr int kPerWave = 4;
  const int item = blockIdx.x;  // bh * nb + I
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = qb * block;
  const int rows = min(block, n - r0);
  const bool ok0 = lane < rows;
  const bool ok1 = block == 128 && lane + 64 < rows;
  const float* ref = rowref + (size_t)bh * n + r0 + lane;
  const float ref0 = ok0 ? ref[0] : 0.f;
  const float ref1 = ok1 ? ref[64] : 0.f;
  const float* base = rowsum + (size_t)bh * nb * n + r0 + lane;
  const float inv_rows = 1.0f / (float)rows;
  for (int kb0 = wave * kPerWave; kb0 < nb; kb0 += 4 * kPerWave) {
    float e[kPerWave];
#pragma unroll
    for (int u = 0; u < kPerWave; ++u) {
      const int kb = kb0 + u;
      float x = 0.f;
      if (kb < nb) {
        const float* src = base + (size_t)kb * n;
        if (ok0) x = __builtin_amdgcn_exp2f(src[0] - ref0);
        if (ok1) x += __builtin_amdgcn_exp2f(src[64] - ref1);
      }
      e[u] = x;
    }
#pragma unroll
    for (int u = 0; u < kPerWave; ++u) e[u] = wave_sum(e[u]);
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < kPerWave; ++u)
        if (kb0 + u < nb) mass[(size_t)item * nb + kb0 + u] = e[u] * inv_rows;
    }
  }
}

hipError_t launch_mass_fold(const float* rowsum, const float* rowref, float* mass, int32_t n,
                            int32_t nb, int32_t block, int32_t bh_count, hipStream_t stream) {
  const long long items = (long long)bh_count * nb;
  hipLaunchKernelGGL(mass_fold_kernel, dim3((unsigned)items), dim3(256), 0, stream, rowsum,
                     rowref, mass, n, nb, block);
  return hipGetLastError();
}

}  // namespace losa
