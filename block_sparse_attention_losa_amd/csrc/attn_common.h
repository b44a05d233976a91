// Pieces of the bf16 attention kernels (attn_bf16.hip): LDS tile swizzles,
// the LDS-DMA load, the transposing LDS read and the union of frozen lists.
#pragma once

#include "losa_device.h"
#include "losa_launch.h"

namespace losa {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// XOR swizzles of the 16-byte chunk index c of row r.
template <int D>
__device__ __forceinline__ int swz_k(int r, int c) {
  constexpr int rows256 = 256 / (2 * D), cpr = D / 8;
  return c ^ ((r / rows256) & (cpr - 1));
}
template <int D>
__device__ __forceinline__ int swz_v(int r, int c) {
  constexpr int rows256 = 256 / (2 * D), groups = D / 32;  // 64-byte groups per row
  return c ^ (((r / rows256) & (groups - 1)) << 2);
}

// Online-softmax reference max: probabilities are exp2(s - m) with
// s - m < kRaise; the reference moves (and O is rescaled) only past that.
constexpr float kRaise = 16.0f;

__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// One wave-wide 16-byte-per-lane load from a buffer straight into 1 KB of
// LDS at lds_addr (lane i lands at lds_addr + 16 i).  Written as inline asm
// so that the compiler does not serialise it against unrelated LDS reads;
// callers wait with vmcnt and a barrier before reading the destination.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned lds_addr, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory", "m0");
}

__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned lds_addr_of(const void* p) {
  return (unsigned)(uintptr_t)p;
}

__device__ __forceinline__ v4i16 ds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

// LDS poisoning, compiled in only for the debug build (LOSA_LDS_POISON):
// every thread of the workgroup fills bytes (a multiple of 16) of LDS at p
// with all-ones words -- NaN as fp32 and as bf16, -1 as an index -- and the
// workgroup then meets at a barrier.  The attention kernels poison all of
// their LDS at the start of each walk over the tiles and every tile slot
// before a load refills it, so that a read of LDS no load or store wrote
// since (a missing wait, a wrong slot, a row past the tile) puts NaN in the
// outputs instead of a stale value that looks plausible.  In other builds
// LOSA_POISON expands to nothing, so their code is untouched.
#ifdef LOSA_LDS_POISON
template <int kThreads>
__device__ __forceinline__ void lds_poison(unsigned char* p, int bytes) {
  const u32x4 ones = {~0u, ~0u, ~0u, ~0u};
  for (int j = threadIdx.x; j < bytes / 16; j += kThreads) ((u32x4*)p)[j] = ones;
  __syncthreads();
}
#define LOSA_POISON(threads, p, bytes) lds_poison<threads>((p), (bytes))
#else
#define LOSA_POISON(threads, p, bytes) ((void)0)
#endif

// Union of the frozen lists of up to kQPW query blocks, ascending, written
// to list[] as (block | member_bits << 16); returns its length.  Called by
// all kThreads threads of the workgroup; nb <= kMaxLen.
template <int kQPW, int kThreads = 256, int kMaxLen = 1024>
__device__ int build_union_list(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                                size_t row0, int nrows, int nb, int* flag, int* list,
                                int* ccount) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nchunks = (nb + 63) >> 6;
  constexpr int kWaves = kThreads / 64;
  constexpr int kPer = (kMaxLen + kThreads - 1) / kThreads;  // entries per thread and row
  for (int j = tid; j < nchunks * 64; j += kThreads) flag[j] = 0;
  // every entry this thread handles is loaded before any is used, so the
  // loads overlap instead of each waiting on the one before it
  int ent[kQPW][kPer];
#pragma unroll
  for (int q = 0; q < kQPW; ++q) {
    const int c = q < nrows ? min(max(cnt[row0 + q], 0), nb) : 0;  // never read past the row
    const int32_t* row = idx + (row0 + q) * nb;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int t = tid + r * kThreads;
      ent[q][r] = t < c ? row[t] : -1;
    }
  }
  __syncthreads();  // flags zeroed
#pragma unroll
  for (int q = 0; q < kQPW; ++q)
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int j = ent[q][r];
      if ((unsigned)j < (unsigned)nb) atomicOr(&flag[j], 1 << q);
    }
  __syncthreads();
  for (int c = wave; c < nchunks; c += kWaves) {
    const unsigned long long m = __ballot(flag[c * 64 + lane] != 0);
    if (lane == 0) ccount[c] = __popcll(m);
  }
  __syncthreads();
  int total = 0;
  for (int c = 0; c < nchunks; ++c) total += ccount[c];
  for (int c = wave; c < nchunks; c += kWaves) {
    int base = 0;
    for (int c2 = 0; c2 < c; ++c2) base += ccount[c2];
    const int f = flag[c * 64 + lane];
    const unsigned long long m = __ballot(f != 0);
    if (f != 0) {
      const unsigned long long below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
      list[base + __popcll(below)] = (c * 64 + lane) | (f << 16);
    }
  }
  __syncthreads();
  return total;
}

}  // namespace losa
