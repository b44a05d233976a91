// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "losa.h"

namespace losa {

// Validation of a descriptor shared by the entry points (losa_api.cpp):
// LOSA_OK and *nb_out = ceil(N / block), or the status to return.
losa_status check_desc(const losa_attn_desc* d, int32_t* nb_out);

// kDenseMass: the dense pass that also writes, per row and key block, the
// block's share of the row's softmax sum (see attn_bf16.hip) for the mass map.
enum Mode : int { kDense = 0, kSparse = 1, kLse = 2, kMass = 3, kDenseMass = 4 };

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;    // sparse: [B*H*nb, nb]
  const int32_t* cnt;    // sparse: [B*H*nb]
  void* o;               // dense/sparse: [B,H,N,D]
  float* lse;            // dense/sparse/lse: [B,H,N] output, may be null (not for kLse)
  const float* lse_in;   // mass: [B,H,N] input
  float* mass;           // mass: [B*H*nb, nb]
  float* rowsum;         // dense+mass: [B*H, nb, N] log2 block sums (workspace)
  float* rowref;         // dense+mass: [B*H, N] per-row offsets (workspace)
  const int32_t* order;  // sparse: workgroup b runs work item order[b] (a plan), or null
  // element strides (batch, head, token; the head dim is contiguous) of Q, K
  // and V, and of O: D*N*H, D*N, D for [B,H,N,D]; D*H*N, D, D*H for [B,N,H,D]
  long long stride_b, stride_h, stride_n;
  long long o_stride_b, o_stride_h, o_stride_n;
  int32_t heads;         // H (to split the (batch, head) index)
  int32_t n;             // tokens
  int32_t nb;            // blocks per sequence
  int32_t items;         // B*H*nb work items (one per query block)
  float scale;           // softmax scale c
};

// Raises kern's dynamic-LDS limit to `bytes` on the current device, once
// per device: the limit is a per-device attribute of the kernel, so a
// process that launches on several GPUs sets it on each.  `done` is the
// calling kernel's own flag array (one flag per device id).
constexpr int kMaxDevices = 64;
template <typename Kernel>
hipError_t set_lds_limit(Kernel kern, int bytes, std::atomic<bool> (&done)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices)
    done[dev].store(true, std::memory_order_release);
  return e;
}

// Launches one pass over every (batch, head, query block).  dtype: 0 bf16,
// 1 fp32.  Returns the HIP status of the launch.
hipError_t launch_attn(int mode, int dtype, int head_dim, int block, const AttnParams& p,
                       hipStream_t stream);

// Query rows per workgroup of a bf16 attention pass.  The dense passes at
// D = 128 that write lse (and the one-sweep construction) use 256 rows (8
// waves, one workgroup per CU): every K/V tile then feeds twice the rows,
// halving the L2 traffic per flop (measured 2-3 % faster).  Dense attention
// without lse runs the 128-row lean pass of sparse attention (attn_bf16.hip)
// and takes the same time.  Sparse attention stays at 128 rows: its
// workgroup walks the union of its query blocks' lists, which is ~3 % longer
// than each list for two 64-token blocks and ~8 % for four.  A sparse work
// item -- and a launch-plan entry -- covers this many rows of one (batch,
// head).
constexpr int attn_rows(int mode, int head_dim, int block, bool lse = true) {
  return (((mode == kDense && lse) || mode == kDenseMass) && head_dim == 128 && block <= 128)
             ? 256
             : 128;
}

// bf16 kernels (LDS-DMA pipeline); same contract as launch_attn.
hipError_t launch_attn_bf16(int mode, int head_dim, int block, const AttnParams& p,
                            hipStream_t stream);

// Folds the per-row block sums of the dense+mass pass into the mass map:
// mass[bh, I, J] = (1/|I|) sum_{i in I} exp2(rowsum[bh, J, i] - rowref[bh, i]).
hipError_t launch_mass_fold(const float* rowsum, const float* rowref, float* mass, int32_t n,
                            int32_t nb, int32_t block, int32_t bh_count, hipStream_t stream);

// taus == nullptr: every row uses tau; otherwise row r uses
// taus[r / rows_per_tau].
hipError_t launch_select(int32_t rows, int32_t nkb, const float* mass, double tau,
                         const double* taus, int32_t rows_per_tau, int32_t* idx, int32_t* count,
                         hipStream_t stream);

// Dispatch order for the sparse kernel: the work items (bh * wph + w, one per
// group of qpw query blocks) ranked by descending cost, cost = the largest
// count among the group's query blocks, laid out per XCD (frozen_lists.hip).
// order: a header of kPlanHeader int32 words {kPlanMagic, n_items, nb, qpw}
// naming the shape the plan was made for, then sparse_plan_slots(n_items)
// slots (n_items = bh_count * wph), -1 in unused slots.  The sparse kernel
// follows the slots only when the header matches its own shape.
constexpr int kPlanHeader = 4;
constexpr int32_t kPlanMagic = 0x4153'6F4C;  // "LoSA"
long long sparse_plan_slots(long long n_items);
hipError_t launch_sparse_plan(const int32_t* count, int32_t nb, int32_t qpw, int32_t bh_count,
                              int32_t* order, hipStream_t stream);

// mask[r, j] = 1 when j is among idx[r, 0:count[r]], else 0 ([rows, nkb] uint8).
hipError_t launch_block_mask(int32_t rows, int32_t nkb, const int32_t* idx, const int32_t* count,
                             uint8_t* mask, hipStream_t stream);

// retained[bh, I] = (1/|I|) sum_{i in I} exp(lse_kept[bh, i] - lse_dense[bh, i]).
hipError_t launch_retained_mass(const float* lse_kept, const float* lse_dense, float* retained,
                                int32_t n, int32_t nb, int32_t block, int32_t bh_count,
                                hipStream_t stream);

}  // namespace losa
