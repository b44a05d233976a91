// bf16 attention passes of the LoSA hot path, written for gfx950 (CDNA4):
//   kDense  - softmax attention over every key block (dense baseline and the
//             construction step's first pass), writes O and lse;
//   kSparse - the same over the frozen key-block list of each query block;
//   kLse    - the row log-sum-exp alone (first pass of the mass map);
//   kMass   - second pass of the mass map: recompute the scores, take
//             exp(s - lse) and sum each (query block, key block) tile.
//
// One workgroup (4 waves) owns one query block of BQ = block rows; each
// wave owns 32 rows.  With 64-row blocks the two waves of a row group split
// every 64-key tile in halves and merge their softmax states at the end.
//
// Data movement is CDNA4-native:
//  * K and V tiles (64 keys) go from HBM straight into LDS with buffer loads
//    in LDS mode (no VGPR staging, no LDS store instructions); rows past the
//    sequence end read as zero through the buffer range check;
//  * tiles are stored row-major with an XOR swizzle of their 16-byte chunks
//    so that both the K fragment reads (ds_read_b128) and the transposing V
//    reads (ds_read_b64_tr_b16, which hand each lane four keys of one head
//    dim) are free of bank conflicts;
//  * K runs one tile ahead of V: the scores of tile t+1 are computed on the
//    matrix cores while tile t's softmax runs on the VALU, and the loads of
//    K(t+2) and V(t+1) are in flight during both.
//
// Scores are computed transposed, S^T = K Q^T, on 32x32x16 MFMA tiles: a
// lane then holds one query row and 16 of the 32 keys of a chunk, so row
// maxima and sums need one cross-half exchange, and the probabilities
// already sit in the B-operand layout of O^T += V^T P^T.  The K rows fed to
// the A operand are permuted (bits 2 and 3 of the row swapped) so that each
// lane's eight probabilities of a 16-key slice are consecutive keys.
#include "losa_device.h"
#include "losa_launch.h"

namespace losa {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int D, int BQ, int MODE>
struct GeoB {
  static constexpr bool kWithV = (MODE == kDense || MODE == kSparse);
  static constexpr int kRG = BQ / 32;          // row groups of 32 rows
  static constexpr int kKS = 4 / kRG;          // waves sharing a row group
  static constexpr int kCPW = 2 / kKS;         // 32-key chunks per wave per tile
  static constexpr int kSubs = BQ / 64;        // 64-key tiles per key block
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTileBytes = 64 * kRowBytes;
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kRowsPer256 = 256 / kRowBytes;   // rows sharing one bank sweep
  static constexpr int kBlocksPerTile = kTileBytes / 1024;  // 1 KB per wave-wide load
  static constexpr int kBlocksPerWave = kBlocksPerTile / 4;
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  static constexpr int kMaxBlocks = 1024;
  static constexpr int kRingBytes = (kWithV ? 4 : 2) * kTileBytes;  // 2 K + 2 V tiles
  static constexpr int kAuxBytes =
      MODE == kSparse ? (2 * kMaxBlocks + 16) * 4 : (MODE == kMass ? 4 * kMaxBlocks * 4 : 0);
  static constexpr int kCombineBytes = (kKS == 2) ? kRG * (2 + (kWithV ? D : 0)) * 32 * 4 : 0;
  static_assert(kCombineBytes <= kRingBytes, "combine buffer must fit in the ring");
  static constexpr int kLdsBytes = kRingBytes + kAuxBytes;
};

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

__device__ int build_ascending_list_b(const int32_t* __restrict__ idx_row, int cnt, int nb,
                                      int* flag, int* list, int* ccount) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nchunks = (nb + 63) >> 6;
  for (int j = tid; j < nchunks * 64; j += 256) flag[j] = 0;
  __syncthreads();
  for (int t = tid; t < cnt; t += 256) {
    const int j = idx_row[t];
    if ((unsigned)j < (unsigned)nb) flag[j] = 1;
  }
  __syncthreads();
  for (int c = wave; c < nchunks; c += 4) {
    const unsigned long long m = __ballot(flag[c * 64 + lane] != 0);
    if (lane == 0) ccount[c] = __popcll(m);
  }
  __syncthreads();
  int total = 0;
  for (int c = 0; c < nchunks; ++c) total += ccount[c];
  for (int c = wave; c < nchunks; c += 4) {
    int base = 0;
    for (int c2 = 0; c2 < c; ++c2) base += ccount[c2];
    const bool f = flag[c * 64 + lane] != 0;
    const unsigned long long m = __ballot(f);
    if (f) {
      const unsigned long long below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
      list[base + __popcll(below)] = c * 64 + lane;
    }
  }
  __syncthreads();
  return total;
}

template <int D, int BQ, int MODE>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(AttnParams p) {
  using G = GeoB<D, BQ, MODE>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int item = xcd_item(blockIdx.x);
  if (item >= p.items) return;  // padding of the XCD-aware grid
  const int nb = p.nb, N = p.n;
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const bf16* __restrict__ qh = (const bf16*)p.q + head_off;
  const bf16* __restrict__ kh = (const bf16*)p.k + head_off;
  const bf16* __restrict__ vh = (const bf16*)p.v + head_off;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int rg = wave % G::kRG, ks = wave / G::kRG;
  const int row = qb * BQ + rg * 32 + l32;
  const bool row_ok = row < N;

  // ---- key blocks visited, in ascending order
  int nblk = nb;
  const int* list = nullptr;
  if constexpr (MODE == kSparse) {
    int* flag = (int*)(smem + G::kRingBytes);
    int* lst = flag + G::kMaxBlocks;
    int* ccount = lst + G::kMaxBlocks;
    const size_t r = (size_t)bh * nb + qb;
    const int cnt = min(max(p.cnt[r], 0), nb);  // never read past the row
    nblk = build_ascending_list_b(p.idx + r * nb, cnt, nb, flag, lst, ccount);
    list = lst;
  }
  float* part = nullptr;  // kMass: per-wave partial tile sums [4][nb]
  if constexpr (MODE == kMass) {
    part = (float*)(smem + G::kRingBytes);
    for (int j = tid; j < 4 * G::kMaxBlocks; j += 256) part[j] = 0.f;
  }
  auto block_at = [&](int t) -> int {
    if constexpr (MODE == kSparse) {
      return list[t];
    } else {
      return t;
    }
  };
  int ntile = nblk * G::kSubs;
  if (G::kSubs == 2 && nblk > 0 && block_at(nblk - 1) == nb - 1 && (nb - 1) * BQ + 64 >= N)
    --ntile;  // empty second half of a short last block
  auto key0_of = [&](int t) -> int {
    const int blk = __builtin_amdgcn_readfirstlane(block_at(G::kSubs == 1 ? t : (t >> 1)));
    return blk * BQ + (G::kSubs == 1 ? 0 : (t & 1) * 64);
  };

  // ---- Q^T as the B operand, in registers
  bf16x8 qreg[D / 16];
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qh, N * G::kRowBytes);
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk)
      qreg[dk] = __builtin_bit_cast(bf16x8, buf_load16(qr, row * G::kRowBytes + dk * 32 + g * 16));
  }

  // ---- LDS ring: K tiles at slots 0/1, V tiles at slots 2/3
  unsigned char* kslot[2] = {smem, smem + G::kTileBytes};
  unsigned char* vslot[2] = {smem + 2 * G::kTileBytes, smem + 3 * G::kTileBytes};

  // per-lane source offsets (inside a tile) of this wave's 1 KB blocks
  int koff[G::kBlocksPerWave], voff[G::kBlocksPerWave];
#pragma unroll
  for (int j = 0; j < G::kBlocksPerWave; ++j) {
    const int b = wave * G::kBlocksPerWave + j;
    const int r = b * G::kRowsPerBlock + lane / G::kChunksPerRow;
    const int pc = lane % G::kChunksPerRow;
    koff[j] = r * G::kRowBytes + swz_k<D>(r, pc) * 16;
    voff[j] = r * G::kRowBytes + swz_v<D>(r, pc) * 16;
  }
  auto dma_tile = [&](const bf16* src, int key0, unsigned char* slot, const int* off) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc((const unsigned char*)src + (size_t)key0 * G::kRowBytes,
                  (N - key0) * G::kRowBytes);
    // wave-uniform LDS destination (M0 must come from a scalar register)
    const unsigned base = __builtin_amdgcn_readfirstlane(lds_addr_of(slot) + wave * G::kBlocksPerWave * 1024);
#pragma unroll
    for (int j = 0; j < G::kBlocksPerWave; ++j) dma16(rs, base + j * 1024, off[j]);
  };

  // ---- per-row running state
  constexpr int kORegs = G::kWithV ? D / 32 : 1;
  f32x16 oacc[kORegs];
#pragma unroll
  for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mt][i] = 0.f;
  float m_run = -INFINITY;  // reference max (log2 domain) of the exp2 arguments
  float l_run = 0.f;        // this lane's partial row sum
  const float c2 = p.scale * kLog2e;
  float lse_row = 0.f;      // kMass: the row's lse (natural), +inf on padding rows
  if constexpr (MODE == kMass) lse_row = row_ok ? p.lse_in[(size_t)bh * N + row] : INFINITY;

  // S^T of this wave's chunks of the K tile in `slot`
  const int prow = perm_row(l32);
  auto compute_s = [&](const unsigned char* slot, f32x16 (&sc)[G::kCPW]) {
#pragma unroll
    for (int cc = 0; cc < G::kCPW; ++cc) {
      const int chunk = G::kKS == 2 ? ks : cc;
      const int r = chunk * 32 + prow;
      const unsigned char* krow = slot + r * G::kRowBytes;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[cc][i] = 0.f;
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk) {
        const bf16x8 a = *(const bf16x8*)(krow + swz_k<D>(r, 2 * dk + g) * 16);
        sc[cc] = mfma_bf16(a, qreg[dk], sc[cc]);
      }
    }
  };

  // V^T operand rows: lane (l%16) of quarter q = l/16 reads 8 bytes of key
  // row kbase + (l%16)/4 (+4 for the upper four keys) at head dims
  // mt*32 + (q%2)*16 + ((l%16)%4)*4 and receives four keys of head dim
  // mt*32 + (q%2)*16 + l%16.
  const int tr_row = (lane & 15) >> 2;
  const int tr_half = ((lane >> 4) & 1) * 16;
  const int tr_col = (lane & 3) * 4;
  auto v_operand = [&](const unsigned char* slot, int kbase, int mt) -> bf16x8 {
    const int d = mt * 32 + tr_half + tr_col;
    const int c = d >> 3, sub = (d & 7) * 2;
    const int r0 = kbase + tr_row, r1 = r0 + 4;
    const v4i16 lo = ds_read_tr16(slot + r0 * G::kRowBytes + swz_v<D>(r0, c) * 16 + sub);
    const v4i16 hi = ds_read_tr16(slot + r1 * G::kRowBytes + swz_v<D>(r1, c) * 16 + sub);
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 w = {l2[0], l2[1], h2[0], h2[1]};
    return __builtin_bit_cast(bf16x8, w);
  };

  auto step = [&](int t, f32x16 (&sc)[G::kCPW], f32x16 (&sn)[G::kCPW]) {
    const int key0 = key0_of(t);
    // loads for later tiles: K(t+2) into the K slot freed by tile t, V(t+1)
    // into the V slot freed by tile t-1
    if (t + 2 < ntile) dma_tile(kh, key0_of(t + 2), kslot[t & 1], koff);
    if constexpr (G::kWithV)
      if (t + 1 < ntile) dma_tile(vh, key0_of(t + 1), vslot[(t + 1) & 1], voff);
    if (t + 1 < ntile) compute_s(kslot[(t + 1) & 1], sn);
    if (key0 + 64 > N) {
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc) {
        const int chunk = G::kKS == 2 ? ks : cc;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + chunk * 32 + perm_row(c_row(i, g)) >= N) sc[cc][i] = -INFINITY;
      }
    }
    if constexpr (MODE == kMass) {
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][i], p.scale, -lse_row) * kLog2e);
      acc = wave_sum(acc);
      if (lane == 0) part[wave * G::kMaxBlocks + (key0 / BQ)] += acc;
    } else {
      // online softmax; the reference max is raised only when a probability
      // could exceed 2^8
      float mx = -INFINITY;
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[cc][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_cand = mx * c2;
      const bool raise = m_cand > m_run + 8.0f;
      const float m_new = raise ? m_cand : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      float pr[G::kCPW][16];
      float lsum = 0.f;
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pr[cc][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][i], c2, -m_use));
          lsum += pr[cc][i];
        }
      l_run = __builtin_fmaf(l_run, alpha, lsum);
      m_run = m_new;
      if constexpr (G::kWithV) {
        if (__ballot(raise)) {
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mt][i] *= alpha;
        }
        const unsigned char* vs = vslot[t & 1];
#pragma unroll
        for (int cc = 0; cc < G::kCPW; ++cc) {
          const int chunk = G::kKS == 2 ? ks : cc;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 pk;
            pk[0] = pack_bf16x2(pr[cc][8 * h + 0], pr[cc][8 * h + 1]);
            pk[1] = pack_bf16x2(pr[cc][8 * h + 2], pr[cc][8 * h + 3]);
            pk[2] = pack_bf16x2(pr[cc][8 * h + 4], pr[cc][8 * h + 5]);
            pk[3] = pack_bf16x2(pr[cc][8 * h + 6], pr[cc][8 * h + 7]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
            for (int mt = 0; mt < kORegs; ++mt) {
              const bf16x8 a = v_operand(vs, chunk * 32 + h * 16 + g * 8, mt);
              oacc[mt] = mfma_bf16(a, pb, oacc[mt]);
            }
          }
        }
      }
    }
    wait_dma_all();
    __syncthreads();
  };

  f32x16 sa[G::kCPW], sb[G::kCPW];
  if (ntile > 0) {
    dma_tile(kh, key0_of(0), kslot[0], koff);
    if constexpr (G::kWithV) dma_tile(vh, key0_of(0), vslot[0], voff);
    if (ntile > 1) dma_tile(kh, key0_of(1), kslot[1], koff);
    wait_dma_all();
    __syncthreads();
    compute_s(kslot[0], sa);
    __syncthreads();  // K slot 0 may be refilled from here on
  }
  for (int t = 0; t < ntile; t += 2) {
    step(t, sa, sb);
    if (t + 1 < ntile) step(t + 1, sb, sa);
  }

  // ------------------------------------------------------------ epilogue
  if constexpr (MODE == kMass) {
    __syncthreads();
    const float inv_rows = 1.0f / (float)min(BQ, N - qb * BQ);
    float* out = p.mass + ((size_t)bh * nb + qb) * nb;
    for (int j = tid; j < nb; j += 256) {
      const float t = (part[j] + part[G::kMaxBlocks + j]) +
                      (part[2 * G::kMaxBlocks + j] + part[3 * G::kMaxBlocks + j]);
      out[j] = t * inv_rows;
    }
    return;
  } else {
    float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    float m_fin = m_run;
    if constexpr (G::kKS == 2) {
      // merge the two key halves of each row group through LDS
      __syncthreads();
      float* cb = (float*)smem + rg * (2 + (G::kWithV ? D : 0)) * 32;
      if (ks == 1) {
        if (g == 0) {
          cb[l32] = m_run;
          cb[32 + l32] = l_tot;
        }
        if constexpr (G::kWithV) {
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) cb[64 + (mt * 32 + c_row(i, g)) * 32 + l32] = oacc[mt][i];
        }
      }
      __syncthreads();
      if (ks == 1) return;
      const float m1 = cb[l32], l1 = cb[32 + l32];
      const float mm = fmaxf(m_run, m1);
      const float a0 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
      const float a1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      l_tot = a0 * l_tot + a1 * l1;
      m_fin = mm;
      if constexpr (G::kWithV) {
#pragma unroll
        for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            oacc[mt][i] = a0 * oacc[mt][i] + a1 * cb[64 + (mt * 32 + c_row(i, g)) * 32 + l32];
      }
    }
    if (!row_ok) return;
    const bool empty = !(l_tot > 0.f);
    if (p.lse != nullptr && g == 0) {
      p.lse[(size_t)bh * N + row] =
          empty ? -INFINITY : (m_fin + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    if constexpr (G::kWithV) {
      const float inv = empty ? 0.f : 1.0f / l_tot;
      bf16* orow = (bf16*)p.o + head_off + (size_t)row * D;
#pragma unroll
      for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = mt * 32 + 8 * i4 + 4 * g;
          u32x2 w = {pack_bf16x2(oacc[mt][4 * i4 + 0] * inv, oacc[mt][4 * i4 + 1] * inv),
                     pack_bf16x2(oacc[mt][4 * i4 + 2] * inv, oacc[mt][4 * i4 + 3] * inv)};
          *(u32x2*)(orow + d0) = w;
        }
    }
  }
}

template <int D, int BQ, int MODE>
hipError_t launch_b(const AttnParams& p, hipStream_t stream) {
  using G = GeoB<D, BQ, MODE>;
  auto kern = attn_bf16_kernel<D, BQ, MODE>;
  static hipError_t attr = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               G::kLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(xcd_grid(p.items)), dim3(256), G::kLdsBytes, stream, p);
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_b_mode(int mode, const AttnParams& p, hipStream_t stream) {
  switch (mode) {
    case kDense: return launch_b<D, BQ, kDense>(p, stream);
    case kSparse: return launch_b<D, BQ, kSparse>(p, stream);
    case kLse: return launch_b<D, BQ, kLse>(p, stream);
    case kMass: return launch_b<D, BQ, kMass>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bf16(int mode, int head_dim, int block, const AttnParams& p,
                            hipStream_t stream) {
  if (head_dim == 64 && block == 64) return launch_b_mode<64, 64>(mode, p, stream);
  if (head_dim == 64 && block == 128) return launch_b_mode<64, 128>(mode, p, stream);
  if (head_dim == 128 && block == 64) return launch_b_mode<128, 64>(mode, p, stream);
  if (head_dim == 128 && block == 128) return launch_b_mode<128, 128>(mode, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace losa
