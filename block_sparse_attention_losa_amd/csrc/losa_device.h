// Device-side building blocks shared by the LoSA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace losa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32 output tile, bf16 inputs with 16-deep contraction: D = A * B + C.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32];
// register i of lane l holds D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16 output tile, bf16 inputs with 32-deep contraction: D = A * B + C.
// Lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16];
// register i of lane l holds D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same output tile, fp32 inputs with a 2-deep contraction: lane l supplies
// A[l%32][l/32] and B[l/32][l%32].
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (within a 32-row tile) held by register i of a lane in half g.
__device__ __forceinline__ constexpr int c_row(int i, int g) {
  return 8 * (i >> 2) + 4 * g + (i & 3);
}

// The values of x in lanes l mod 32 and l mod 32 + 32 (lower half first),
// in every lane l, without an LDS round trip: v_permlane32_swap exchanges
// the upper 32 lanes of its first operand with the lower 32 lanes of its
// second (lane layout checked with a probe), so with x in both operands the
// first holds (x_lo, x_lo) and the second (x_hi, x_hi) afterwards.  Written
// as inline asm with both registers as in/out operands: the compiler's
// builtin for it returned the first register for both results.  The s_nop
// covers the VALU-write -> permlane-read hazard on the inputs; fetch-inactive
// is set in case the exchange ends up in a branch that runs half the wave.
__device__ __forceinline__ void lane_halves(float x, float& lo, float& hi) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32_e64 %0, %1 fi:1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}
// x[l mod 32] + x[l mod 32 + 32], the same bits in both lanes of a pair.
__device__ __forceinline__ float pair_sum(float x) {
  float lo, hi;
  lane_halves(x, lo, hi);
  return lo + hi;
}
// The max is taken inside the same asm block: fmaxf on the asm outputs
// would first canonicalize both (two more VALU ops on the softmax's path).
__device__ __forceinline__ float pair_max(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32_e64 %0, %1 fi:1\n\ts_nop 0\n\tv_max_f32 %0, %0, %1"
      : "+v"(a), "+v"(b));
  return a;
}

// The 32-bit value held by lane l ^ LJ, LJ in {1, 2, 4, 8}, all within a
// 16-lane row: distances 1 and 2 are quad permutations, 4 a mirror of each
// 8-lane half row (lane i reads i ^ 7) followed by a quad reversal (i ^ 3),
// 8 a rotation of the row by 8.
template <int LJ>
__device__ __forceinline__ int row_xor(int v) {
  static_assert(LJ == 1 || LJ == 2 || LJ == 4 || LJ == 8, "lane distance inside a DPP row");
  if constexpr (LJ == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  if constexpr (LJ == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  if constexpr (LJ == 4)
    return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true), 0x1B,
                                    0xF, 0xF, true);
  return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);
}

template <int LJ>
__device__ __forceinline__ float row_xor(float v) {
  return __int_as_float(row_xor<LJ>(__float_as_int(v)));
}

template <int LJ>
__device__ __forceinline__ double row_xor(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = row_xor<LJ>((int)(unsigned)u), hi = row_xor<LJ>((int)(unsigned)(u >> 32));
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Sum over the 16 lanes of the row, the same bits in every lane (a
// butterfly: each lane adds the same pairs, and float addition commutes).
__device__ __forceinline__ float row_sum16(float x) {
  x += row_xor<1>(x);
  x += row_xor<2>(x);
  x += row_xor<4>(x);
  return x + row_xor<8>(x);
}

// Sum over the 64 lanes, the same bits in every lane: the butterfly inside
// each 16-lane row, the two half-waves added (v_permlane32_swap), then the
// two rows of a half read out and added -- VALU and DPP work only, where a
// ds_bpermute butterfly makes six LDS round trips in a row.
__device__ __forceinline__ float wave_sum(float x) {
  x = pair_sum(row_sum16(x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
  return x;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero, which is how the kernels read the ragged last block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Workgroup -> work item.  Workgroups are handed to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8).  Each XCD is given the same contiguous
// slice of query blocks -- [x*per, (x+1)*per) with per = ceil(nb/8) -- of
// every (batch, head), heads in order: neighbouring query blocks, whose
// key-block lists overlap, share one L2, every XCD sees the same mix of
// cheap and expensive heads, and a head's K/V is live in all L2s at once.
constexpr int kXcds = 8;
__host__ __device__ __forceinline__ int xcd_slice(int nb) { return (nb + kXcds - 1) / kXcds; }
__host__ __device__ __forceinline__ int xcd_grid(int nb, int bh_count) {
  return kXcds * xcd_slice(nb) * bh_count;
}
// Returns the work item (bh * nb + qb) of workgroup b, or -1 for padding.
__device__ __forceinline__ int xcd_item(int b, int nb, int bh_count) {
  const int per = xcd_slice(nb);
  const int x = b % kXcds, k = b / kXcds;
  const int bh = k / per, qb = x * per + (k - (k / per) * per);
  return (bh < bh_count && qb < nb) ? bh * nb + qb : -1;
}

}  // namespace losa
