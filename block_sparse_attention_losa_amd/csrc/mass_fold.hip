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

namespace {

// The four stored values of rows row .. row+3 of the query block (`rows` of
// them exist).  kFull: all exist and rows start at multiples of four floats,
// so one 16-byte load; otherwise rows past the block read as 0 (they get an
// infinite reference below, so they add nothing).
template <bool kFull>
__device__ __forceinline__ float4 load4(const float* __restrict__ src, int row, int rows) {
  if constexpr (kFull) {
    return *(const float4*)src;
  } else {
    float4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < rows) v.x = src[0];
    if (row + 1 < rows) v.y = src[1];
    if (row + 2 < rows) v.z = src[2];
    if (row + 3 < rows) v.w = src[3];
    return v;
  }
}

// The mass row of one (batch*head, query block): see mass_fold_kernel.
template <int CHUNKS, bool kFull>
__device__ __forceinline__ void fold_item(const float* __restrict__ rowsum,
                                          const float* __restrict__ rowref,
                                          float* __restrict__ mass, int n, int nb, int item,
                                          int bh, int r0, int rows) {
  constexpr int kU = 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, q = lane & 15;
  float ref[CHUNKS][4];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int row = c * 64 + 4 * q;
    const float4 r = load4<kFull>(rowref + (size_t)bh * n + r0 + row, row, rows);
    ref[c][0] = row < rows ? r.x : INFINITY;
    ref[c][1] = row + 1 < rows ? r.y : INFINITY;
    ref[c][2] = row + 2 < rows ? r.z : INFINITY;
    ref[c][3] = row + 3 < rows ? r.w : INFINITY;
  }
  const float* base = rowsum + (size_t)bh * nb * n + r0 + 4 * q;
  const float inv_rows = 1.0f / (float)rows;
  for (int j0 = wave * 4 * kU; j0 < nb; j0 += 16 * kU) {
    float4 val[kU][CHUNKS];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kb = j0 + 4 * u + grp;
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) {
        val[u][c] = float4{0.f, 0.f, 0.f, 0.f};
        if (kb < nb) val[u][c] = load4<kFull>(base + (size_t)kb * n + c * 64, c * 64 + 4 * q, rows);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) {
        s += __builtin_amdgcn_exp2f(val[u][c].x - ref[c][0]);
        s += __builtin_amdgcn_exp2f(val[u][c].y - ref[c][1]);
        s += __builtin_amdgcn_exp2f(val[u][c].z - ref[c][2]);
        s += __builtin_amdgcn_exp2f(val[u][c].w - ref[c][3]);
      }
      s = row_sum16(s);
      const int kb = j0 + 4 * u + grp;
      if (q == 0 && kb < nb) mass[(size_t)item * nb + kb] = s * inv_rows;
    }
  }
}

}  // namespace

// One workgroup (four waves) per (batch*head, query block I).  A load
// instruction of a wave covers four key blocks: lanes 16g .. 16g+15 take key
// block J0 + g, lane q of them rows 4q .. 4q+3 of each 64-row chunk of I with
// one 16-byte load, and four such loads are issued before any is used.  A
// block's row sum is the lane's own values, then a butterfly over the 16
// lanes of the DPP row -- a fixed order, so the result is deterministic.
// (A whole-wave reduction per key block through ds_bpermute, with four
// blocks in flight per wave, reached about a third of HBM bandwidth.)
template <int CHUNKS>
__global__ void __launch_bounds__(256) mass_fold_kernel(const float* __restrict__ rowsum,
                                                        const float* __restrict__ rowref,
                                                        float* __restrict__ mass, int n, int nb) {
  const int item = blockIdx.x;  // bh * nb + I
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const int r0 = qb * 64 * CHUNKS;
  const int rows = min(64 * CHUNKS, n - r0);
  // 16-byte loads: every row of the block present, row starts at multiples
  // of four floats
  const bool full = rows == 64 * CHUNKS && (n & 3) == 0 &&
                    (((uintptr_t)rowsum | (uintptr_t)rowref) & 15) == 0;
  if (full)
    fold_item<CHUNKS, true>(rowsum, rowref, mass, n, nb, item, bh, r0, rows);
  else
    fold_item<CHUNKS, false>(rowsum, rowref, mass, n, nb, item, bh, r0, rows);
}

hipError_t launch_mass_fold(const float* rowsum, const float* rowref, float* mass, int32_t n,
                            int32_t nb, int32_t block, int32_t bh_count, hipStream_t stream) {
  const long long items = (long long)bh_count * nb;
  if (block == 64) {
    hipLaunchKernelGGL(mass_fold_kernel<1>, dim3((unsigned)items), dim3(256), 0, stream, rowsum,
                       rowref, mass, n, nb);
  } else if (block == 128) {
    hipLaunchKernelGGL(mass_fold_kernel<2>, dim3((unsigned)items), dim3(256), 0, stream, rowsum,
                       rowref, mass, n, nb);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace losa
