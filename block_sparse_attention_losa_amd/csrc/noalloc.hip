// losa_block_mass_noalloc: the two-pass mass map (losa_block_mass without a
// caller lse) for callers that cannot allocate device memory -- code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
// The first pass's row log-sum-exp goes to a scratch array that the library
// holds in its own code object (one per GPU, allocated when the module
// loads, kept until the process ends); the call itself allocates nothing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "losa.h"
#include "losa_launch.h"

namespace {

// B*H*N row log-sum-exps of the first pass, fp32: 16 MiB per GPU.
__device__ __align__(256) float scratch[LOSA_NOALLOC_MAX_ROWS];

// Device address of `scratch` per device, looked up on the first call made
// with that device current (in host code the array's name is only a host
// stand-in for the symbol, never an address a kernel may use).
std::mutex scratch_mu;
float* scratch_ptr[losa::kMaxDevices] = {};

losa_status device_scratch(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= losa::kMaxDevices)
    return LOSA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    float* ptr = nullptr;
    if (hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch)) != hipSuccess ||
        ptr == nullptr)
      return LOSA_ERR_DEVICE;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return LOSA_OK;
}

}  // namespace

extern "C" losa_status losa_block_mass_noalloc(const losa_attn_desc* desc, const void* q,
                                               const void* k, float* mass, void* stream) {
  int32_t nb = 0;
  const losa_status st = losa::check_desc(desc, &nb);
  if (st != LOSA_OK) return st;
  const int64_t rows = static_cast<int64_t>(desc->batch) * desc->heads * desc->seq_len;
  if (rows > LOSA_NOALLOC_MAX_ROWS) return LOSA_ERR_SCRATCH_LIMIT;
  if (!q || !k || !mass) return LOSA_ERR_NULL_POINTER;
  float* lse = nullptr;
  const losa_status dst = device_scratch(&lse);
  if (dst != LOSA_OK) return dst;
  // every row's lse is written by the first pass before the second reads
  // it, so nothing has to be cleared between calls
  return losa_block_mass(desc, q, k, nullptr, lse, mass, stream);
}
