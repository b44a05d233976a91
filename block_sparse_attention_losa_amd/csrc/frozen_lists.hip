// Small kernels over the frozen block lists:
//  * block_mask_kernel -- the lists as a dense mask tensor (query block x key
//    block, 1 = retained), the form in which the pages store the selection
//    for reuse (ubos.tech blog, "How It Works in Practice", Phase 2);
//  * retained_mass_kernel -- how much of a later step's dense attention mass
//    the frozen lists still cover, from the row log-sum-exps of a sparse pass
//    (lse') and a dense pass (lse) on the same inputs:
//      R[I] = (1/|I|) sum_{i in I} exp(lse'_i - lse_i),
//    since exp(lse'_i - lse_i) = sum_{j kept} exp(s_ij) / sum_j exp(s_ij).
//    The pages report that the high-mass block set stays stable across
//    denoising steps (ubos.tech blog, "Key Findings"; aitobox blog, "Key
//    Highlights"); R measures that on the caller's own inputs;
//  * sparse_plan_kernel -- a dispatch order for the sparse kernel, made once
//    per set of frozen lists: the work items ranked by descending cost and
//    dealt to the XCDs so that every XCD gets the same mix of long and short
//    items and runs its longest ones first (layout below).
//    Per-head kept fractions range from a few percent to all blocks, and in
//    the default head-major order the last items to start are often long
//    ones, leaving the chip part-idle at the end.
// All are memory-bound or tiny; none allocates.
#include "losa_device.h"
#include "losa_launch.h"

namespace losa {

// One wave per row of the mask, four rows per workgroup.  The row is built
// as byte flags in LDS (zero, then one per listed block; entries outside
// [0, nkb) and past count are ignored) and written out coalesced.
__global__ void __launch_bounds__(256) block_mask_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ count,
                                                         uint8_t* __restrict__ mask, int rows,
                                                         int nkb) {
  __shared__ unsigned char flags[4][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  const bool live = row < rows;
  unsigned char* f = flags[wave];
  for (int j = lane; j < nkb; j += 64) f[j] = 0;
  __syncthreads();
  if (live) {
    const int c = min(max(count[row], 0), nkb);
    const int32_t* list = idx + (size_t)row * nkb;
    for (int t = lane; t < c; t += 64) {
      const int j = list[t];
      if ((unsigned)j < (unsigned)nkb) f[j] = 1;
    }
  }
  __syncthreads();
  if (live) {
    uint8_t* out = mask + (size_t)row * nkb;
    for (int j = lane; j < nkb; j += 64) out[j] = f[j];
  }
}

// One wave per (batch*head, query block): lane l takes rows l and l + 64 of
// the block; a butterfly sums them in a fixed order.
__global__ void __launch_bounds__(256) retained_mass_kernel(const float* __restrict__ lse_kept,
                                                            const float* __restrict__ lse_dense,
                                                            float* __restrict__ retained, int n,
                                                            int nb, int block, int items) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wave;  // bh * nb + I
  if (item >= items) return;  // no barriers: whole waves leave together
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const int r0 = qb * block;
  const int rows = min(block, n - r0);
  const size_t base = (size_t)bh * n + r0;
  float acc = 0.f;
  for (int r = lane; r < rows; r += 64)
    acc += expf(lse_kept[base + r] - lse_dense[base + r]);
  acc = wave_sum(acc);
  if (lane == 0) retained[item] = acc / (float)rows;
}

// Plan layout.  Items are ranked by cost, descending, in kPlanBuckets
// buckets (cost * kPlanBuckets / (nb + 1)); within a bucket they keep their
// index order (head-major, query blocks ascending), so runs of consecutive
// ranks are neighbouring query blocks of one head, whose lists overlap.
// Runs of kPlanChunk ranks go to one XCD, runs dealt to the 8 XCDs in turn:
// rank s -> chunk c = s / kPlanChunk, XCD x = c % 8, round r = c / 8, and
// slot 8 * (r * kPlanChunk + s % kPlanChunk) + x, which the hardware hands
// to XCD x as its (r * kPlanChunk + s % kPlanChunk)-th workgroup.  Every XCD
// thus gets the same mix of costs, longest first, and the workgroups
// resident on an XCD mostly share one head's K/V.  Slots past the last item
// hold -1.  (On the Wan2.1-1.3B lists this keeps the simulated makespan
// within 3 % of the balanced bound; sorting by exact cost reaches 1 % but
// scatters each head's query blocks and doubled the K/V traffic.)
constexpr int kPlanBuckets = 32;
constexpr int kPlanChunk = 8;

__host__ __device__ inline long long plan_slots(long long n_items) {
  const long long chunks = (n_items + kPlanChunk - 1) / kPlanChunk;
  return (long long)kXcds * kPlanChunk * ((chunks + kXcds - 1) / kXcds);
}

__device__ __forceinline__ int plan_slot(int s) {
  const int c = s / kPlanChunk;
  return kXcds * ((c / kXcds) * kPlanChunk + s % kPlanChunk) + c % kXcds;
}

// One workgroup of 1024 threads: a stable counting sort of the items by
// bucket (histogram, then tiles of 1024 items in index order, ranks within a
// tile from wave ballots), written straight to the slots.  Deterministic.
__global__ void __launch_bounds__(1024) sparse_plan_kernel(const int32_t* __restrict__ count,
                                                           int nb, int qpw, int n_items, int wph,
                                                           int32_t* __restrict__ order) {
  __shared__ int start[kPlanBuckets];       // next rank of each bucket
  __shared__ int wcnt[16][kPlanBuckets];    // per-wave bucket counts of a tile
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto bucket_of = [&](int item) -> int {
    const int bh = item / wph;
    const int w = item - bh * wph;
    const int q0 = w * qpw;
    int c = 0;
    for (int q = q0; q < min(nb, q0 + qpw); ++q)
      c = max(c, min(max(count[(size_t)bh * nb + q], 0), nb));
    return min(kPlanBuckets - 1, c * kPlanBuckets / (nb + 1));
  };
  if (tid < kPlanBuckets) start[tid] = 0;
  __syncthreads();
  for (int item = tid; item < n_items; item += 1024) atomicAdd(&start[bucket_of(item)], 1);
  __syncthreads();
  if (tid == 0) {  // exclusive prefix, most expensive bucket first
    int run = 0;
    for (int k = kPlanBuckets - 1; k >= 0; --k) {
      const int h = start[k];
      start[k] = run;
      run += h;
    }
  }
  // slots of the last round that no rank reaches
  const int slots = (int)plan_slots(n_items);
  for (int j = tid; j < kXcds * kPlanChunk; j += 1024) {
    const int slot = slots - kXcds * kPlanChunk + j;
    const int x = slot % kXcds, within = slot / kXcds;
    const int s_rank = ((within / kPlanChunk) * kXcds + x) * kPlanChunk + within % kPlanChunk;
    if (s_rank >= n_items) order[slot] = -1;
  }
  __syncthreads();
  for (int base = 0; base < n_items; base += 1024) {
    const int item = base + tid;
    const int bkt = item < n_items ? bucket_of(item) : -1;
    const unsigned long long below = lane ? ((~0ull) >> (64 - lane)) : 0ull;
    int rank = 0;
    for (int k = 0; k < kPlanBuckets; ++k) {
      const unsigned long long m = __ballot(bkt == k);
      if (bkt == k) rank = __popcll(m & below);
      if (lane == 0) wcnt[wave][k] = __popcll(m);
    }
    __syncthreads();
    if (bkt >= 0) {
      int s_rank = start[bkt] + rank;
      for (int w2 = 0; w2 < wave; ++w2) s_rank += wcnt[w2][bkt];
      order[plan_slot(s_rank)] = item;
    }
    __syncthreads();
    if (tid < kPlanBuckets) {
      int add = 0;
      for (int w2 = 0; w2 < 16; ++w2) add += wcnt[w2][tid];
      start[tid] += add;
    }
    __syncthreads();
  }
}

long long sparse_plan_slots(long long n_items) { return plan_slots(n_items); }

hipError_t launch_sparse_plan(const int32_t* count, int32_t nb, int32_t qpw, int32_t bh_count,
                              int32_t* order, hipStream_t stream) {
  if (nb > 1024 || qpw < 1) return hipErrorInvalidValue;
  const int wph = (nb + qpw - 1) / qpw;
  hipLaunchKernelGGL(sparse_plan_kernel, dim3(1), dim3(1024), 0, stream, count, nb, qpw,
                     bh_count * wph, wph, order);
  return hipGetLastError();
}

hipError_t launch_block_mask(int32_t rows, int32_t nkb, const int32_t* idx, const int32_t* count,
                             uint8_t* mask, hipStream_t stream) {
  if (nkb > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_mask_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     idx, count, mask, rows, nkb);
  return hipGetLastError();
}

hipError_t launch_retained_mass(const float* lse_kept, const float* lse_dense, float* retained,
                                int32_t n, int32_t nb, int32_t block, int32_t bh_count,
                                hipStream_t stream) {
  const long long items = (long long)bh_count * nb;
  hipLaunchKernelGGL(retained_mass_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0,
                     stream, lse_kept, lse_dense, retained, n, nb, block, (int)items);
  return hipGetLastError();
}

}  // namespace losa
