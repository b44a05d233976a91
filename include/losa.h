/*
 * losa.h -- C-ABI of the LoSA attention hot path for AMD Instinct MI355X
 * (gfx950).
 *
 * LoSA (arXiv 2608.12032) measures exact block attention masses at one early
 * dense denoising step, keeps for every head and query block the smallest
 * set of key/value blocks whose mass reaches a threshold (0.99 by default),
 * and reuses those frozen block lists for block-sparse attention at every
 * later step (mlsanity.com paper index, "Abstract (arXiv)"; legiblepapers,
 * "Summary & Methodology Analysis" and FAQ Q4-Q6; ubos.tech blog, "How It
 * Works in Practice", Phases 1-3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors Q, K, V, O are [B, H, N, D] (D fastest) in device memory,
 *    element type bf16 or fp32 (losa_dtype), 16-byte aligned: contiguous by
 *    default, or (bf16) laid out by the strides in losa_attn_desc, e.g. the
 *    [B, N, H, D] layout a DiT projection produces, read in place.  lse is [B, H, N] fp32, natural log.  mass is [B, H, nb, nb]
 *    fp32 (key block fastest); idx is [B, H, nb, nb] int32 and count
 *    [B, H, nb] int32.  nb = ceil(N / block); the last block holds the
 *    N - (nb-1)*block remaining tokens.  fp32/int32 arrays must be 4-byte
 *    aligned.
 *  - Every pointer argument is a device pointer owned by the caller; the
 *    library never allocates, frees or synchronises and may be called from
 *    several host threads at once.  Its only state is set once per kernel
 *    and device on first use: the kernel's dynamic-LDS limit
 *    (hipFuncSetAttribute), and for losa_block_mass_noalloc the address of
 *    its scratch array.  Outputs must not overlap inputs.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Work is enqueued asynchronously on it, as kernel launches only (no
 *    memset or copy), so calls on different streams may run concurrently
 *    and calls can be captured into a HIP graph and replayed; make one call
 *    of each entry point on the device before capturing, so that the
 *    first-use attribute is not set inside the capture.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    status other than LOSA_OK means nothing was launched.  A launch the HIP
 *    runtime rejects returns LOSA_ERR_DEVICE.  Faults while the kernels run
 *    surface at the caller's next synchronisation, as for any HIP kernel.
 *  - Limits: D in {64, 128}; block in {64, 128}; nb <= LOSA_MAX_BLOCKS;
 *    B*H*nb < 2^31.
 */
#ifndef LOSA_H
#define LOSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOSA_MAX_BLOCKS 1024

typedef enum {
  LOSA_OK = 0,
  LOSA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL                 */
  LOSA_ERR_BAD_SHAPE = 2,      /* sizes outside the supported set           */
  LOSA_ERR_BAD_DTYPE = 3,      /* unknown element type                      */
  LOSA_ERR_BAD_THRESHOLD = 4,  /* threshold NaN or <= 0                     */
  LOSA_ERR_MISALIGNED = 5,     /* pointer alignment below the requirement   */
  LOSA_ERR_DEVICE = 6,         /* the HIP runtime rejected a launch         */
  LOSA_ERR_BAD_ARGUMENT = 7,   /* other invalid argument (e.g. scale)       */
  LOSA_ERR_WORKSPACE = 8,      /* workspace smaller than required           */
  LOSA_ERR_SCRATCH_LIMIT = 9   /* B*H*N above LOSA_NOALLOC_MAX_ROWS          */
} losa_status;

typedef enum { LOSA_BF16 = 0, LOSA_FP32 = 1 } losa_dtype;

/* Shape of one attention layer call. */
typedef struct {
  int32_t batch;     /* B >= 1                                            */
  int32_t heads;     /* H >= 1                                            */
  int32_t seq_len;   /* N >= 1, tokens of the flattened 3D sequence       */
  int32_t head_dim;  /* D, 64 or 128                                      */
  int32_t block;     /* square block size (query and key), 64 or 128      */
  int32_t dtype;     /* losa_dtype of Q, K, V and O                        */
  float scale;       /* softmax scale c; 0 selects 1/sqrt(D)              */
  /* Element strides between batch items, heads and tokens (the D elements of
   * a token are contiguous) of Q, K and V (shared) and of O.  A triple of 0s
   * means contiguous [B, H, N, D].  Otherwise (bf16 only): token stride >= D,
   * every stride a multiple of 8 elements (16 bytes) and >= 0, and
   * (N-1)*token_stride*2 + 2*D < 2^31; the stride of a dimension of size 1
   * is ignored.  Examples: [B, N, H, D] is (N*H*D, D, H*D); Q of a packed
   * [B, N, 3, H, D] projection is (3*N*H*D, D, 3*H*D).  lse, mass, idx and
   * count stay contiguous.  An O layout in which two output elements could
   * share an address (ordered by stride, each dimension of size > 1 must step
   * past the extent of those inside it) is rejected with
   * LOSA_ERR_BAD_ARGUMENT. */
  int64_t stride_batch;
  int64_t stride_head;
  int64_t stride_token;
  int64_t o_stride_batch;
  int64_t o_stride_head;
  int64_t o_stride_token;
} losa_attn_desc;

/* ceil(seq_len / block), or -1 when desc is NULL or block < 1. */
int32_t losa_num_blocks(const losa_attn_desc* desc);

/*
 * Dense softmax attention over all N keys: the pass the sampler runs at its
 * first denoising steps and at the construction step (legiblepapers,
 * "Summary & Methodology Analysis"; mlsanity.com, "Abstract (arXiv)").
 *   s_ij = c <q_i, k_j>,  lse_i = log sum_j exp(s_ij),
 *   o_i  = sum_j exp(s_ij - lse_i) v_j.
 * q, k, v: inputs [B,H,N,D]; o: output [B,H,N,D] (same dtype);
 * lse: output [B,H,N] fp32, or NULL to skip it.
 */
losa_status losa_dense_attn(const losa_attn_desc* desc, const void* q, const void* k,
                            const void* v, void* o, float* lse, void* stream);

/*
 * Exact block attention mass (the "mass map") of the construction step
 * (mlsanity.com, "Abstract (arXiv)": exact block attention masses at one
 * early dense step; ubos.tech blog, "How It Works in Practice", Phase 1):
 *   M[b,h,I,J] = (1/|I|) sum_{i in I} sum_{j in J} exp(s_ij - lse_i)
 * with |I| the valid rows of query block I.  Each row of M sums to 1.
 * lse: the dense pass's row log-sum-exp [B,H,N]; when NULL, a first pass
 *      computes it into lse_scratch ([B,H,N] fp32, then required).
 * mass: output [B,H,nb,nb] fp32.
 */
losa_status losa_block_mass(const losa_attn_desc* desc, const void* q, const void* k,
                            const float* lse, float* lse_scratch, float* mass,
                            void* stream);

/*
 * losa_block_mass with lse = NULL, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The first pass's row log-sum-exp goes to a scratch
 * array of LOSA_NOALLOC_MAX_ROWS floats (16 MiB) that the library keeps in
 * each GPU's memory for the life of the process; the call allocates and
 * frees nothing.  Requires B*H*N <= LOSA_NOALLOC_MAX_ROWS, else
 * LOSA_ERR_SCRATCH_LIMIT (nothing launched).  The scratch is shared by every
 * call on a GPU: calls that overlap on one GPU (different streams or host
 * threads) race on it and must be ordered by the caller.  The first call on
 * a device looks the array's address up (hipGetSymbolAddress); make one call
 * before capturing it into a graph.  mass: output [B,H,nb,nb] fp32, the
 * same bits as losa_block_mass.
 */
#define LOSA_NOALLOC_MAX_ROWS 4194304
losa_status losa_block_mass_noalloc(const losa_attn_desc* desc, const void* q, const void* k,
                                    float* mass, void* stream);

/*
 * The construction step in one sweep over the keys: dense attention (as
 * losa_dense_attn) and the block mass map (as losa_block_mass) of the same
 * inputs.  The pages measure exact block masses at one early dense step and
 * put the cost of that step at about one denoising step (mlsanity.com,
 * "Abstract (arXiv)"; ubos.tech blog, "How It Works in Practice", Phase 1).
 * Here the dense pass also records, for each row and key block, the block's
 * share of the row's softmax sum (log2, against a per-row reference) in
 * `workspace`, and a second, memory-bound kernel folds those into M once the
 * row sums are final: the scores are computed once, not twice.
 *   M[b,h,I,J] = (1/|I|) sum_{i in I} sum_{j in J} exp(s_ij - lse_i)
 * equals the two-pass result up to rounding.
 * o: output [B,H,N,D]; lse: output [B,H,N] fp32 or NULL; mass: output
 * [B,H,nb,nb] fp32.
 * workspace: device memory, 256-byte aligned, owned by the caller; its
 *   contents on entry are ignored and on return are unspecified.  With
 *   losa_dense_attn_mass_workspace(desc) bytes (4*B*H*N*(nb+1) plus
 *   alignment: 0.8 GB for B1 H12 N32760 block 64, 10.6 GB for B1 H24
 *   N118800 block 128) every (b, h) runs in one pass.  Any smaller size of
 *   at least losa_dense_attn_mass_workspace_min(desc) bytes (one (b, h):
 *   4*N*(nb+1) plus alignment, 67 MB and 442 MB for those two shapes) is
 *   also accepted: the call then makes several passes, each over as many
 *   heads of one batch item as the workspace holds, with the same results
 *   bit for bit.  Calls running at the same time need separate workspaces.
 * For LOSA_FP32 the call runs the dense pass and the two-pass mass kernel
 * (the workspace then holds lse when lse is NULL).
 * Returns LOSA_ERR_WORKSPACE when workspace_bytes is below the minimum.
 */
int64_t losa_dense_attn_mass_workspace(const losa_attn_desc* desc);
int64_t losa_dense_attn_mass_workspace_min(const losa_attn_desc* desc);
losa_status losa_dense_attn_mass(const losa_attn_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float* lse, float* mass,
                                 void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Threshold selection (ubos.tech blog, "How It Works in Practice", Phase 2;
 * mlsanity.com, "Abstract (arXiv)"; legiblepapers, FAQ Q4).  For each of the
 * `rows` rows of `mass` ([rows, nkb] fp32, finite and >= 0): order the key
 * blocks by descending mass, ties by ascending block index; accumulate the
 * masses in that order in float64; count = the smallest k whose running sum
 * reaches `threshold` (>=), or nkb when none does or threshold >= 1.
 * idx: output [rows, nkb] int32; entries [0, count) hold the kept blocks in
 *      that order, later entries are left untouched.
 * count: output [rows] int32.
 * Requires 1 <= nkb <= LOSA_MAX_BLOCKS, rows >= 1, threshold > 0 (not NaN).
 * For the [B,H,nb,nb] mass map, rows = B*H*nb and nkb = nb.
 */
losa_status losa_select(int32_t rows, int32_t nkb, const float* mass, double threshold,
                        int32_t* idx, int32_t* count, void* stream);

/*
 * losa_select with a threshold per row or per group of rows, for retained-
 * mass targets that vary by head or by query block (ubos.tech blog, "What
 * Comes Next": adapting the retained-mass target per frame or scene).  Row r
 * uses thresholds[r / rows_per_threshold]: with the [B,H,nb,nb] mass map,
 * rows_per_threshold = nb gives one threshold per (b,h) and 1 one per query
 * block.  thresholds: device array of ceil(rows / rows_per_threshold)
 * doubles, 8-byte aligned.  The values are read on the device and so are not
 * validated: >= 1 (or NaN) keeps every block, <= 0 keeps one.
 * Other arguments and results as losa_select.  rows_per_threshold >= 1.
 */
losa_status losa_select_per_row(int32_t rows, int32_t nkb, const float* mass,
                                const double* thresholds, int32_t rows_per_threshold,
                                int32_t* idx, int32_t* count, void* stream);

/*
 * The frozen lists as a mask tensor, the form in which the pages store the
 * selection for reuse (ubos.tech blog, "How It Works in Practice", Phase 2:
 * a mask of shape (heads, query blocks, key blocks)).
 *   mask[r, j] = 1 if j is among idx[r, 0:count[r]], else 0.
 * idx: [rows, nkb] int32, count: [rows] int32 (as from losa_select; entries
 * outside [0, nkb) are ignored, count is clamped to [0, nkb]);
 * mask: output [rows, nkb] uint8, no alignment needed.
 */
losa_status losa_block_mask(int32_t rows, int32_t nkb, const int32_t* idx, const int32_t* count,
                            uint8_t* mask, void* stream);

/*
 * Drift diagnostic of the frozen lists: the share of a later step's dense
 * attention mass that the lists still cover, per query block.  The pages
 * report that the high-mass block set stays stable across denoising steps
 * (ubos.tech blog, "Key Findings"; aitobox blog, "Key Highlights"); this
 * measures it without a mass pass:
 *   R[b,h,I] = (1/|I|) sum_{i in I} exp(lse'_i - lse_i)
 *            = (1/|I|) sum_{i in I} sum_{j kept} exp(s_ij - lse_i),
 * lse_kept: the lse output [B,H,N] of losa_sparse_attn on the step's inputs;
 * lse_dense: the lse output [B,H,N] of losa_dense_attn on the same inputs;
 * retained: output [B,H,nb] fp32.  A query block with an empty list gets 0.
 */
losa_status losa_retained_mass(const losa_attn_desc* desc, const float* lse_kept,
                               const float* lse_dense, float* retained, void* stream);

/*
 * Block-sparse attention over frozen block lists (ubos.tech blog, "How It
 * Works in Practice", Phase 3; legiblepapers, "Summary & Methodology
 * Analysis": later steps attend only to the retained keys).  For query
 * block I of (b,h) the retained keys are the tokens of blocks
 * idx[b,h,I,0:count[b,h,I]]; the softmax is renormalised over them:
 *   lse'_i = log sum_{j kept} exp(s_ij),  o_i = sum_{j kept} exp(s_ij - lse'_i) v_j.
 * idx/count as produced by losa_select; the lists may be in any order.
 * Lists that did not come from losa_select (a file, another tool) are safe
 * to pass: count is clamped to [0, nb], entries outside [0, nb) are
 * ignored and a repeated entry counts once, so no list makes the kernel
 * read outside Q, K, V or the list row.  A query block whose list ends up
 * empty gets o = 0 and lse' = -inf.
 * o: output [B,H,N,D]; lse: output [B,H,N] fp32 or NULL.
 */
losa_status losa_sparse_attn(const losa_attn_desc* desc, const void* q, const void* k,
                             const void* v, const int32_t* idx, const int32_t* count,
                             void* o, float* lse, void* stream);

/*
 * Launch plan for block-sparse attention over a fixed set of frozen lists.
 * The lists do not change after the construction step (mlsanity.com,
 * "Abstract (arXiv)": index freezing; legiblepapers, FAQ Q6), and neither
 * does the work they imply, so the order in which the GPU should run it can
 * be fixed once too: per-head kept fractions range from a few percent to
 * every block, and running the work items longest-first, in runs of
 * neighbouring query blocks spread over the chip's 8 XCDs so that each XCD
 * gets the same summed cost, keeps all compute units busy to the end.
 * losa_sparse_plan writes that order (int32, losa_sparse_plan_size(desc)
 * bytes, 4-byte aligned, caller-owned) from count [B,H,nb]; only count is
 * read.  Recompute it whenever count changes.  Returns LOSA_ERR_WORKSPACE
 * when plan_bytes is below the size.  The same counts give the same plan;
 * results do not depend on the order.  The
 * plan opens with a header naming the shape it was made for (work items,
 * nb, query blocks per item).
 * losa_sparse_attn_planned computes exactly what losa_sparse_attn computes
 * (bit-identical outputs) in the plan's order.  plan_bytes below
 * losa_sparse_plan_size(desc) returns LOSA_ERR_WORKSPACE (nothing
 * launched).  A plan whose header names another shape is not followed: the
 * kernel then runs the work items in index order, so the results are still
 * complete and correct, only the launch is slower.  A plan made from other
 * counts of the same shape is still a complete order, only a slower one.
 * Slot entries are trusted: an entry outside the valid range (a plan
 * overwritten by the caller) is skipped, leaving its rows unwritten.  For
 * LOSA_FP32 the plan is ignored.
 */
int64_t losa_sparse_plan_size(const losa_attn_desc* desc);
losa_status losa_sparse_plan(const losa_attn_desc* desc, const int32_t* count, int32_t* plan,
                             int64_t plan_bytes, void* stream);
losa_status losa_sparse_attn_planned(const losa_attn_desc* desc, const void* q, const void* k,
                                     const void* v, const int32_t* idx, const int32_t* count,
                                     const int32_t* plan, int64_t plan_bytes, void* o,
                                     float* lse, void* stream);

/* Static text for a status code. */
const char* losa_status_string(losa_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t losa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOSA_H */
