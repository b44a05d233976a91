// C-ABI of the LoSA hot path: argument validation and dispatch to the
// kernels.  Every check happens before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "losa.h"
#include "losa_launch.h"

namespace {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// True when no two elements of a [B, H, N, D] view with these element
// strides (D contiguous) share an address: taken innermost first by stride,
// every dimension of size > 1 must step past the whole extent of the
// dimensions inside it.  (Sufficient, and exact for the permuted and sliced
// layouts a caller hands in.)
bool disjoint(const losa_attn_desc* d, int64_t sb, int64_t sh, int64_t sn) {
  int64_t size[3] = {d->batch, d->heads, d->seq_len}, stride[3] = {sb, sh, sn};
  for (int i = 0; i < 3; ++i)  // order by stride, ascending
    for (int j = i + 1; j < 3; ++j)
      if (stride[j] < stride[i]) {
        const int64_t ts = stride[i], tz = size[i];
        stride[i] = stride[j];
        size[i] = size[j];
        stride[j] = ts;
        size[j] = tz;
      }
  int64_t extent = d->head_dim;
  for (int i = 0; i < 3; ++i) {
    if (size[i] == 1) continue;
    if (stride[i] < extent) return false;
    extent += stride[i] * (size[i] - 1);
  }
  return true;
}

}  // namespace

namespace losa {

losa_status check_desc(const losa_attn_desc* d, int32_t* nb_out) {
  if (d == nullptr) return LOSA_ERR_NULL_POINTER;
  if (d->dtype != LOSA_BF16 && d->dtype != LOSA_FP32) return LOSA_ERR_BAD_DTYPE;
  if (d->batch < 1 || d->heads < 1 || d->seq_len < 1) return LOSA_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return LOSA_ERR_BAD_SHAPE;
  if (d->block != 64 && d->block != 128) return LOSA_ERR_BAD_SHAPE;
  const int64_t nb = (static_cast<int64_t>(d->seq_len) + d->block - 1) / d->block;
  if (nb > LOSA_MAX_BLOCKS) return LOSA_ERR_BAD_SHAPE;
  const int64_t items = static_cast<int64_t>(d->batch) * d->heads * nb;
  if (items >= (int64_t{1} << 31)) return LOSA_ERR_BAD_SHAPE;
  if (!std::isfinite(d->scale) || d->scale < 0.f) return LOSA_ERR_BAD_ARGUMENT;
  if (static_cast<int64_t>(d->seq_len) * d->head_dim * 2 >= (int64_t{1} << 31))
    return LOSA_ERR_BAD_SHAPE;
  for (int t = 0; t < 2; ++t) {
    // the stride of a dimension of size 1 never enters an address
    const int64_t sb = d->batch == 1 ? 0 : (t ? d->o_stride_batch : d->stride_batch);
    const int64_t sh = d->heads == 1 ? 0 : (t ? d->o_stride_head : d->stride_head);
    const int64_t sn = t ? d->o_stride_token : d->stride_token;
    if ((t ? d->o_stride_batch : d->stride_batch) == 0 && (t ? d->o_stride_head : d->stride_head) == 0 &&
        sn == 0)
      continue;  // contiguous
    if (d->dtype != LOSA_BF16) return LOSA_ERR_BAD_ARGUMENT;
    if (sn < d->head_dim || sh < 0 || sb < 0) return LOSA_ERR_BAD_ARGUMENT;
    if (sn % 8 || sh % 8 || sb % 8) return LOSA_ERR_MISALIGNED;
    if ((static_cast<int64_t>(d->seq_len) - 1) * sn * 2 + 2 * d->head_dim >= (int64_t{1} << 31))
      return LOSA_ERR_BAD_SHAPE;
    // outputs must not alias one another (inputs are only read)
    if (t == 1 && !disjoint(d, sb, sh, sn)) return LOSA_ERR_BAD_ARGUMENT;
  }
  *nb_out = static_cast<int32_t>(nb);
  return LOSA_OK;
}

}  // namespace losa

namespace {

using losa::check_desc;

float effective_scale(const losa_attn_desc* d) {
  return d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
}

losa::AttnParams base_params(const losa_attn_desc* d, int32_t nb) {
  losa::AttnParams p{};
  p.n = d->seq_len;
  p.nb = nb;
  p.items = d->batch * d->heads * nb;
  p.scale = effective_scale(d);
  p.heads = d->heads;
  const long long cn = d->head_dim, ch = static_cast<long long>(d->seq_len) * d->head_dim,
                  cb = ch * d->heads;  // contiguous [B, H, N, D]
  const bool in_c = d->stride_batch == 0 && d->stride_head == 0 && d->stride_token == 0;
  const bool out_c = d->o_stride_batch == 0 && d->o_stride_head == 0 && d->o_stride_token == 0;
  // strides of size-1 dimensions are never multiplied by a nonzero index
  p.stride_b = in_c ? cb : (d->batch == 1 ? 0 : d->stride_batch);
  p.stride_h = in_c ? ch : (d->heads == 1 ? 0 : d->stride_head);
  p.stride_n = in_c ? cn : d->stride_token;
  p.o_stride_b = out_c ? cb : (d->batch == 1 ? 0 : d->o_stride_batch);
  p.o_stride_h = out_c ? ch : (d->heads == 1 ? 0 : d->o_stride_head);
  p.o_stride_n = out_c ? cn : d->o_stride_token;
  return p;
}

losa_status device_status(hipError_t e) { return e == hipSuccess ? LOSA_OK : LOSA_ERR_DEVICE; }

// Workspace of losa_dense_attn_mass for a pass over `heads` (b, h) slices:
// the per-row block sums [heads, nb, N] fp32, then the per-row offsets
// [heads, N] fp32 at the next 256-byte boundary.
int64_t rowsum_bytes(const losa_attn_desc* d, int32_t nb, int64_t heads) {
  const int64_t raw = int64_t{4} * heads * nb * d->seq_len;
  return (raw + 255) / 256 * 256;
}
int64_t dense_mass_workspace(const losa_attn_desc* d, int32_t nb, int64_t heads) {
  return rowsum_bytes(d, nb, heads) + int64_t{4} * heads * d->seq_len;
}
int64_t all_heads(const losa_attn_desc* d) { return int64_t{d->batch} * d->heads; }

// Sparse work items: one per workgroup of the sparse kernel, i.e. per
// losa::attn_rows query rows of each (b, h).
int32_t blocks_per_item(const losa_attn_desc* d) {
  return losa::attn_rows(losa::kSparse, d->head_dim, d->block) / d->block;
}
int64_t plan_items(const losa_attn_desc* d, int32_t nb) {
  const int32_t qpw = blocks_per_item(d);
  return int64_t{d->batch} * d->heads * ((nb + qpw - 1) / qpw);
}
int64_t plan_entries(const losa_attn_desc* d, int32_t nb) {
  return losa::kPlanHeader + losa::sparse_plan_slots(plan_items(d, nb));
}

}  // namespace

extern "C" {

int32_t losa_num_blocks(const losa_attn_desc* desc) {
  if (desc == nullptr || desc->block < 1 || desc->seq_len < 0) return -1;
  return static_cast<int32_t>((static_cast<int64_t>(desc->seq_len) + desc->block - 1) /
                              desc->block);
}

losa_status losa_dense_attn(const losa_attn_desc* desc, const void* q, const void* k,
                            const void* v, void* o, float* lse, void* stream) {
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (!q || !k || !v || !o) return LOSA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return LOSA_ERR_MISALIGNED;
  losa::AttnParams p = base_params(desc, nb);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return device_status(losa::launch_attn(losa::kDense, desc->dtype, desc->head_dim, desc->block,
                                         p, static_cast<hipStream_t>(stream)));
}

losa_status losa_block_mass(const losa_attn_desc* desc, const void* q, const void* k,
                            const float* lse, float* lse_scratch, float* mass, void* stream) {
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (!q || !k || !mass || (!lse && !lse_scratch)) return LOSA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(mass, 4) || (lse && !aligned(lse, 4)) ||
      (!lse && !aligned(lse_scratch, 4)))
    return LOSA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  losa::AttnParams p = base_params(desc, nb);
  p.q = q;
  p.k = k;
  if (lse == nullptr) {
    p.lse = lse_scratch;
    st = device_status(
        losa::launch_attn(losa::kLse, desc->dtype, desc->head_dim, desc->block, p, s));
    if (st != LOSA_OK) return st;
    lse = lse_scratch;
  }
  p.lse = nullptr;
  p.lse_in = lse;
  p.mass = mass;
  return device_status(
      losa::launch_attn(losa::kMass, desc->dtype, desc->head_dim, desc->block, p, s));
}

int64_t losa_dense_attn_mass_workspace(const losa_attn_desc* desc) {
  int32_t nb = 0;
  if (check_desc(desc, &nb) != LOSA_OK) return -1;
  return dense_mass_workspace(desc, nb, all_heads(desc));
}

int64_t losa_dense_attn_mass_workspace_min(const losa_attn_desc* desc) {
  int32_t nb = 0;
  if (check_desc(desc, &nb) != LOSA_OK) return -1;
  return dense_mass_workspace(desc, nb, 1);
}

losa_status losa_dense_attn_mass(const losa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float* lse, float* mass,
                                 void* workspace, int64_t workspace_bytes, void* stream) {
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (!q || !k || !v || !o || !mass || !workspace) return LOSA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(mass, 4) || !aligned(workspace, 256) || (lse && !aligned(lse, 4)))
    return LOSA_ERR_MISALIGNED;
  if (workspace_bytes < dense_mass_workspace(desc, nb, 1)) return LOSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const losa::AttnParams base = base_params(desc, nb);
  // Heads per pass: every (b, h) at once when the whole workspace is given;
  // otherwise passes over runs of the heads of one batch item, as many as
  // the workspace holds (the per-row arithmetic is the same either way, so
  // are the results)
  int64_t group = all_heads(desc);
  if (workspace_bytes < dense_mass_workspace(desc, nb, group)) {
    group = desc->heads;
    while (group > 1 && dense_mass_workspace(desc, nb, group) > workspace_bytes) --group;
  }
  const int64_t esize = desc->dtype == LOSA_FP32 ? 4 : 2;
  const int64_t nn = desc->seq_len;
  const int64_t passes_per_batch = group >= all_heads(desc) ? 1 : (desc->heads + group - 1) / group;
  const int32_t batches = group >= all_heads(desc) ? 1 : desc->batch;
  for (int32_t b = 0; b < batches; ++b) {
    for (int64_t pass = 0; pass < passes_per_batch; ++pass) {
      const int64_t h0 = pass * group;
      const int64_t g = group >= all_heads(desc) ? group : std::min<int64_t>(group, desc->heads - h0);
      const int64_t first = int64_t{b} * desc->heads + h0;  // first (b, h) of the pass
      losa::AttnParams p = base;
      if (g < all_heads(desc)) {
        // the pass sees its g heads of batch item b as heads 0..g-1 of one
        // batch item: base pointers moved to head (b, h0), head strides kept
        p.heads = static_cast<int32_t>(g);
        p.items = static_cast<int32_t>(g * nb);
      }
      const int64_t in_off = (b * base.stride_b + h0 * base.stride_h) * esize;
      const int64_t out_off = (b * base.o_stride_b + h0 * base.o_stride_h) * esize;
      p.q = static_cast<const char*>(q) + in_off;
      p.k = static_cast<const char*>(k) + in_off;
      p.v = static_cast<const char*>(v) + in_off;
      p.o = static_cast<char*>(o) + out_off;
      float* lse_g = lse ? lse + first * nn : nullptr;
      float* mass_g = mass + first * nb * nb;
      float* rowsum = static_cast<float*>(workspace);
      float* rowref =
          reinterpret_cast<float*>(static_cast<char*>(workspace) + rowsum_bytes(desc, nb, g));
      if (desc->dtype == LOSA_FP32) {
        // fp32: the dense pass writes lse (into the workspace when the caller
        // wants none) and the two-pass mass kernel reads it
        float* lse_buf = lse_g ? lse_g : rowref;
        p.lse = lse_buf;
        st = device_status(losa::launch_attn(losa::kDense, desc->dtype, desc->head_dim,
                                             desc->block, p, s));
        if (st != LOSA_OK) return st;
        p.o = nullptr;
        p.v = nullptr;
        p.lse = nullptr;
        p.lse_in = lse_buf;
        p.mass = mass_g;
        st = device_status(
            losa::launch_attn(losa::kMass, desc->dtype, desc->head_dim, desc->block, p, s));
        if (st != LOSA_OK) return st;
        continue;
      }
      p.lse = lse_g;
      p.rowsum = rowsum;
      p.rowref = rowref;
      st = device_status(losa::launch_attn(losa::kDenseMass, desc->dtype, desc->head_dim,
                                           desc->block, p, s));
      if (st != LOSA_OK) return st;
      st = device_status(losa::launch_mass_fold(rowsum, rowref, mass_g, desc->seq_len, nb,
                                                desc->block, static_cast<int32_t>(g), s));
      if (st != LOSA_OK) return st;
    }
  }
  return LOSA_OK;
}

losa_status losa_select(int32_t rows, int32_t nkb, const float* mass, double threshold,
                        int32_t* idx, int32_t* count, void* stream) {
  if (!mass || !idx || !count) return LOSA_ERR_NULL_POINTER;
  if (rows < 1 || nkb < 1 || nkb > LOSA_MAX_BLOCKS) return LOSA_ERR_BAD_SHAPE;
  if (std::isnan(threshold) || !(threshold > 0.0)) return LOSA_ERR_BAD_THRESHOLD;
  if (!aligned(mass, 4) || !aligned(idx, 4) || !aligned(count, 4)) return LOSA_ERR_MISALIGNED;
  return device_status(losa::launch_select(rows, nkb, mass, threshold, nullptr, 1, idx, count,
                                          static_cast<hipStream_t>(stream)));
}

losa_status losa_select_per_row(int32_t rows, int32_t nkb, const float* mass,
                                const double* thresholds, int32_t rows_per_threshold,
                                int32_t* idx, int32_t* count, void* stream) {
  if (!mass || !thresholds || !idx || !count) return LOSA_ERR_NULL_POINTER;
  if (rows < 1 || nkb < 1 || nkb > LOSA_MAX_BLOCKS) return LOSA_ERR_BAD_SHAPE;
  if (rows_per_threshold < 1) return LOSA_ERR_BAD_ARGUMENT;
  if (!aligned(mass, 4) || !aligned(thresholds, 8) || !aligned(idx, 4) || !aligned(count, 4))
    return LOSA_ERR_MISALIGNED;
  return device_status(losa::launch_select(rows, nkb, mass, 0.0, thresholds, rows_per_threshold,
                                          idx, count, static_cast<hipStream_t>(stream)));
}

losa_status losa_block_mask(int32_t rows, int32_t nkb, const int32_t* idx, const int32_t* count,
                            uint8_t* mask, void* stream) {
  if (!idx || !count || !mask) return LOSA_ERR_NULL_POINTER;
  if (rows < 1 || nkb < 1 || nkb > LOSA_MAX_BLOCKS) return LOSA_ERR_BAD_SHAPE;
  if (!aligned(idx, 4) || !aligned(count, 4)) return LOSA_ERR_MISALIGNED;
  return device_status(
      losa::launch_block_mask(rows, nkb, idx, count, mask, static_cast<hipStream_t>(stream)));
}

losa_status losa_retained_mass(const losa_attn_desc* desc, const float* lse_kept,
                               const float* lse_dense, float* retained, void* stream) {
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (!lse_kept || !lse_dense || !retained) return LOSA_ERR_NULL_POINTER;
  if (!aligned(lse_kept, 4) || !aligned(lse_dense, 4) || !aligned(retained, 4))
    return LOSA_ERR_MISALIGNED;
  return device_status(losa::launch_retained_mass(lse_kept, lse_dense, retained, desc->seq_len,
                                                  nb, desc->block, desc->batch * desc->heads,
                                                  static_cast<hipStream_t>(stream)));
}

losa_status losa_sparse_attn(const losa_attn_desc* desc, const void* q, const void* k,
                             const void* v, const int32_t* idx, const int32_t* count, void* o,
                             float* lse, void* stream) {
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (!q || !k || !v || !o || !idx || !count) return LOSA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(idx, 4) || !aligned(count, 4) || (lse && !aligned(lse, 4)))
    return LOSA_ERR_MISALIGNED;
  losa::AttnParams p = base_params(desc, nb);
  p.q = q;
  p.k = k;
  p.v = v;
  p.idx = idx;
  p.cnt = count;
  p.o = o;
  p.lse = lse;
  return device_status(losa::launch_attn(losa::kSparse, desc->dtype, desc->head_dim, desc->block,
                                         p, static_cast<hipStream_t>(stream)));
}

int64_t losa_sparse_plan_size(const losa_attn_desc* desc) {
  int32_t nb = 0;
  if (check_desc(desc, &nb) != LOSA_OK) return -1;
  return 4 * plan_entries(desc, nb);
}

losa_status losa_sparse_plan(const losa_attn_desc* desc, const int32_t* count, int32_t* plan,
                             int64_t plan_bytes, void* stream) {
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (!count || !plan) return LOSA_ERR_NULL_POINTER;
  if (!aligned(count, 4) || !aligned(plan, 4)) return LOSA_ERR_MISALIGNED;
  if (plan_bytes < 4 * plan_entries(desc, nb)) return LOSA_ERR_WORKSPACE;
  return device_status(losa::launch_sparse_plan(count, nb, blocks_per_item(desc),
                                                desc->batch * desc->heads, plan,
                                                static_cast<hipStream_t>(stream)));
}

losa_status losa_sparse_attn_planned(const losa_attn_desc* desc, const void* q, const void* k,
                                     const void* v, const int32_t* idx, const int32_t* count,
                                     const int32_t* plan, int64_t plan_bytes, void* o,
                                     float* lse, void* stream) {
  if (plan == nullptr) return LOSA_ERR_NULL_POINTER;
  if (!aligned(plan, 4)) return LOSA_ERR_MISALIGNED;
  int32_t nb = 0;
  losa_status st = check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  if (plan_bytes < 4 * plan_entries(desc, nb)) return LOSA_ERR_WORKSPACE;
  if (!q || !k || !v || !o || !idx || !count) return LOSA_ERR_NULL_POINTER;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(idx, 4) || !aligned(count, 4) || (lse && !aligned(lse, 4)))
    return LOSA_ERR_MISALIGNED;
  losa::AttnParams p = base_params(desc, nb);
  p.q = q;
  p.k = k;
  p.v = v;
  p.idx = idx;
  p.cnt = count;
  p.o = o;
  p.lse = lse;
  if (desc->dtype == LOSA_BF16) p.order = plan;  // the fp32 kernel keeps its own order
  return device_status(losa::launch_attn(losa::kSparse, desc->dtype, desc->head_dim, desc->block,
                                         p, static_cast<hipStream_t>(stream)));
}

const char* losa_status_string(losa_status status) {
  // A C caller may pass any int: read the argument's bits as an int rather
  // than load an out-of-range value of the C++ enum type (undefined there)
  int code = 0;
  static_assert(sizeof(code) == sizeof(status), "losa_status is int-sized");
  std::memcpy(&code, &status, sizeof(code));
  switch (code) {
    case LOSA_OK: return "ok";
    case LOSA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case LOSA_ERR_BAD_SHAPE: return "unsupported sizes (D, block, N, B*H*nb or nkb)";
    case LOSA_ERR_BAD_DTYPE: return "unknown element type";
    case LOSA_ERR_BAD_THRESHOLD: return "threshold must be > 0 and not NaN";
    case LOSA_ERR_MISALIGNED: return "pointer alignment below the requirement";
    case LOSA_ERR_DEVICE: return "the HIP runtime rejected a launch";
    case LOSA_ERR_BAD_ARGUMENT:
      return "invalid argument (scale not finite or negative, bad strides or aliasing output "
             "layout, or rows per threshold < 1)";
    case LOSA_ERR_WORKSPACE: return "workspace smaller than the size the library asks for";
    case LOSA_ERR_SCRATCH_LIMIT:
      return "B*H*N exceeds the library's static scratch (LOSA_NOALLOC_MAX_ROWS rows)";
  }
  return "unknown status";
}

int32_t losa_version(void) { return 200; }

}  // extern "C"
