// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace losa {

enum Mode : int { kDense = 0, kSparse = 1, kLse = 2, kMass = 3 };

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
  int32_t n;             // tokens
  int32_t nb;            // blocks per sequence
  int32_t items;         // B*H*nb work items (one per query block)
  float scale;           // softmax scale c
};

// Launches one pass over every (batch, head, query block).  dtype: 0 bf16,
// 1 fp32.  Returns the HIP status of the launch.
hipError_t launch_attn(int mode, int dtype, int head_dim, int block, const AttnParams& p,
                       hipStream_t stream);

// bf16 kernels (LDS-DMA pipeline); same contract as launch_attn.
hipError_t launch_attn_bf16(int mode, int head_dim, int block, const AttnParams& p,
                            hipStream_t stream);

hipError_t launch_select(int32_t rows, int32_t nkb, const float* mass, double tau,
                         int32_t* idx, int32_t* count, hipStream_t stream);

}  // namespace losa
