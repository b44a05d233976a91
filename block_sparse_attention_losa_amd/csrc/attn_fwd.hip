// fp32 attention passes of the LoSA hot path on gfx950 (CDNA4), for fp32
// inputs (the bf16 passes are in attn_bf16.hip):
//   kDense  - softmax attention over every key block (dense baseline and the
//             construction step's first pass), writes O and lse;
//   kSparse - the same over the frozen key-block list of each query block;
//   kLse    - the row log-sum-exp alone (first pass of the mass map);
//   kMass   - the second pass of the mass map: recompute the scores, take
//             exp(s - lse) and sum each (query block, key block) tile.
//
// One workgroup (4 waves) owns one query block of BQ = block rows.  Key and
// value tiles of 64 keys are staged through LDS, double buffered, with the
// next tile's global loads in flight while the current one is computed.
// Each wave owns 32 query rows; with 64-row query blocks the two waves of a
// row group split every 64-key tile in halves and merge their partial
// softmax states at the end.
//
// Scores are computed transposed, S^T = K Q^T, on 32x32x2 fp32 MFMA tiles:
// a lane then holds one query row and 16 of the 32 keys, so row maxima and
// sums need one cross-half exchange only, and the probabilities already sit
// in the B-operand layout of O^T += V^T P^T.  This path exists for exact
// fp32 inputs (the tiny reference case), not for speed.

#include "losa_device.h"
#include "losa_launch.h"

namespace losa {

template <int D, int BQ, int MODE>
struct Geo {
  static constexpr bool kWithV = (MODE == kDense || MODE == kSparse);
  static constexpr int kThreads = 256;
  static constexpr int kRG = BQ / 32;          // row groups of 32 rows
  static constexpr int kKS = 4 / kRG;          // waves sharing a row group
  static constexpr int kKT = 64;               // keys per staged tile
  static constexpr int kCPW = 2 / kKS;         // 32-key chunks per wave per tile
  static constexpr int kSubs = BQ / 64;        // staged tiles per key block
  static constexpr int kKStr = D + 4;                   // K row stride (elements)
  static constexpr int kVStr = D + 4;                   // V row stride (elements)
  static constexpr int kKBytes = kKT * kKStr * 4;
  static constexpr int kVBytes = kWithV ? kKT * kVStr * 4 : 0;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kStages = 2 * kStage;
  static constexpr int kMaxBlocks = 1024;
  static constexpr int kAuxBytes =
      MODE == kSparse ? (2 * kMaxBlocks + 16) * 4 : (MODE == kMass ? 4 * kMaxBlocks * 4 : 0);
  static constexpr int kCombineBytes = (kKS == 2) ? kRG * (2 + (kWithV ? D : 0)) * 32 * 4 : 0;
  static_assert(kCombineBytes <= kStages, "combine buffer must fit in the stage buffers");
  static constexpr int kLdsBytes = kStages + kAuxBytes;
  // K (and V) chunks of 16 bytes per thread per tile
  static constexpr int kKChunks = kKT * D * 4 / 16 / kThreads;
};

// ---------------------------------------------------------------------------
// Frozen list -> ascending block order in LDS.  Visiting kept blocks in
// ascending order keeps concurrently running query blocks of one head on
// nearby K/V and puts the (possibly partial) last block last.
__device__ int build_ascending_list(const int32_t* __restrict__ idx_row, int cnt, int nb,
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

// ---------------------------------------------------------------------------
// D = 128 needs more than 256 registers per lane: one wave per SIMD.
template <int D, int BQ, int MODE>
__global__ void __launch_bounds__(256, (D == 128 ? 1 : 2)) attn_kernel(AttnParams p) {
  using G = Geo<D, BQ, MODE>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int item = xcd_item(blockIdx.x, p.nb, p.items / p.nb);
  if (item < 0) return;  // padding of the XCD-aware grid
  const int nb = p.nb, N = p.n;
  const int bh = item / nb;
  const int qb = item - bh * nb;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const float* __restrict__ qh = (const float*)p.q + head_off;
  const float* __restrict__ kh = (const float*)p.k + head_off;
  const float* __restrict__ vh = (const float*)p.v + head_off;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int rg = wave % G::kRG, ks = wave / G::kRG;
  const int row = qb * BQ + rg * 32 + l32;
  const bool row_ok = row < N;

  // ---- the key blocks this query block visits, in ascending order
  int nblk = nb;
  const int* list = nullptr;
  if constexpr (MODE == kSparse) {
    int* flag = (int*)(smem + G::kStages);
    int* lst = flag + G::kMaxBlocks;
    int* ccount = lst + G::kMaxBlocks;
    const size_t r = (size_t)bh * nb + qb;
    const int cnt = min(max(p.cnt[r], 0), nb);  // never read past the row
    nblk = build_ascending_list(p.idx + r * nb, cnt, nb, flag, lst, ccount);
    list = lst;
  }
  float* part = nullptr;  // kMass: per-wave partial tile sums [4][nb]
  if constexpr (MODE == kMass) {
    part = (float*)(smem + G::kStages);
    for (int j = tid; j < 4 * G::kMaxBlocks; j += 256) part[j] = 0.f;
    // made visible by the first barrier of the tile loop
  }
  auto block_at = [&](int t) -> int {
    if constexpr (MODE == kSparse) {
      return list[t];
    } else {
      return t;
    }
  };
  int nstage = nblk * G::kSubs;
  if (G::kSubs == 2 && nblk > 0 && block_at(nblk - 1) == nb - 1 && (nb - 1) * BQ + 64 >= N)
    --nstage;  // empty second half of a short last block

  // ---- Q^T as the B operand, kept in registers: lane half g holds head
  // dims g*D/2 .. g*D/2 + D/2 - 1 of its row
  float qreg[D / 2];
  constexpr int kRowBytes = D * 4;
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qh, N * kRowBytes);
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      const u32x4 x = buf_load16(qr, row * kRowBytes + (g * (D / 2) + s) * 4);
      qreg[s] = __uint_as_float(x[0]);
      qreg[s + 1] = __uint_as_float(x[1]);
      qreg[s + 2] = __uint_as_float(x[2]);
      qreg[s + 3] = __uint_as_float(x[3]);
    }
  }

  // ---- stage registers (global -> regs -> LDS); the tile is addressed by a
  // scalar buffer resource starting at its first key
  u32x4 kr[G::kKChunks];
  u32x4 vr[G::kKChunks];
  auto load_k = [&](int key0) {
    const int bytes = (N - key0) * kRowBytes;
    const __amdgpu_buffer_rsrc_t kt =
        make_rsrc((const unsigned char*)kh + (size_t)key0 * kRowBytes, bytes);
#pragma unroll
    for (int j = 0; j < G::kKChunks; ++j) kr[j] = buf_load16(kt, (j * 256 + tid) * 16);
  };
  auto load_v = [&](int key0) {
    if constexpr (G::kWithV) {
      const int bytes = (N - key0) * kRowBytes;
      const __amdgpu_buffer_rsrc_t vt =
          make_rsrc((const unsigned char*)vh + (size_t)key0 * kRowBytes, bytes);
#pragma unroll
      for (int j = 0; j < G::kKChunks; ++j) vr[j] = buf_load16(vt, (j * 256 + tid) * 16);
    }
  };

  // LDS: two K tiles, then two V tiles, both row-major with padded rows
  auto kbuf = [&](int b) -> float* { return (float*)(smem + b * G::kKBytes); };
  auto vbuf = [&](int b) -> float* { return (float*)(smem + 2 * G::kKBytes + b * G::kVBytes); };

  auto store_k = [&](int b) {
    float* klds = kbuf(b);
#pragma unroll
    for (int j = 0; j < G::kKChunks; ++j) {
      const int c = j * 256 + tid;
      const int key = c / (D / 4), col = c % (D / 4);
      *(u32x4*)(klds + key * G::kKStr + col * 4) = kr[j];
    }
  };
  auto store_v = [&](int b) {
    if constexpr (G::kWithV) {
      float* vlds = vbuf(b);
#pragma unroll
      for (int j = 0; j < G::kKChunks; ++j) {
        const int c = j * 256 + tid;
        const int key = c / (D / 4), col = c % (D / 4);
        *(u32x4*)(vlds + key * G::kVStr + col * 4) = vr[j];
      }
    }
  };

  auto key0_of = [&](int s) -> int {
    const int blk = __builtin_amdgcn_readfirstlane(block_at(G::kSubs == 1 ? s : (s >> 1)));
    return blk * BQ + (G::kSubs == 1 ? 0 : (s & 1) * 64);
  };

  // ---- per-row running state
  constexpr int kORegs = G::kWithV ? D / 32 : 0;
  f32x16 oacc[kORegs > 0 ? kORegs : 1];
#pragma unroll
  for (int mt = 0; mt < (kORegs > 0 ? kORegs : 1); ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[mt][i] = 0.f;
  float m_run = -INFINITY;  // reference max (log2 domain) of exp2 arguments
  float l_run = 0.f;        // this lane's partial row sum
  const float c2 = p.scale * kLog2e;
  float lse_row = 0.f;      // kMass: the row's log-sum-exp (natural), +inf for padding rows
  if constexpr (MODE == kMass) lse_row = row_ok ? p.lse_in[(size_t)bh * N + row] : INFINITY;

  // S^T of this wave's chunks of the K tile in buffer b
  auto compute_s = [&](int b, f32x16 (&sc)[G::kCPW]) {
    const float* klds = kbuf(b);
#pragma unroll
    for (int cc = 0; cc < G::kCPW; ++cc) {
      const int chunk = G::kKS == 2 ? ks : cc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[cc][i] = 0.f;
      const float* krow = klds + (chunk * 32 + l32) * G::kKStr;
#pragma unroll
      for (int st = 0; st < D / 2; st += 4) {
        const float4 a = *(const float4*)(krow + g * (D / 2) + st);
        sc[cc] = mfma_f32(a.x, qreg[st], sc[cc]);
        sc[cc] = mfma_f32(a.y, qreg[st + 1], sc[cc]);
        sc[cc] = mfma_f32(a.z, qreg[st + 2], sc[cc]);
        sc[cc] = mfma_f32(a.w, qreg[st + 3], sc[cc]);
      }
    }
  };

  // One pipelined step: the scores of tile t+1 are computed (MFMA) while
  // tile t's scores go through the softmax (VALU); then tile t's P V
  // product; then the next tiles are staged.  K runs one tile ahead of V.
  auto step = [&](int t, f32x16 (&sc)[G::kCPW], f32x16 (&sn)[G::kCPW]) {
    const int key0 = key0_of(t);
    if (t + 1 < nstage) compute_s((t + 1) & 1, sn);
    if (key0 + 64 > N) {
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc) {
        const int chunk = G::kKS == 2 ? ks : cc;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + chunk * 32 + c_row(i, g) >= N) sc[cc][i] = -INFINITY;
      }
    }
    if constexpr (MODE == kMass) {
      // exp(s - lse) summed over this wave's rows and keys of the tile
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][i], p.scale, -lse_row) * kLog2e);
      acc = wave_sum(acc);
      if (lane == 0) part[wave * G::kMaxBlocks + (key0 / BQ)] += acc;
    } else {
      // online softmax with a lazily raised reference max: the reference
      // moves only when a probability could exceed 2^8
      float mx = -INFINITY;
#pragma unroll
      for (int cc = 0; cc < G::kCPW; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[cc][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_cand = mx * c2;
      const bool raise = m_cand > m_run + 8.0f;
      const float m_new = raise ? m_cand : m_run;
      // 0 when m_run = -inf; lanes that keep their reference scale by 1
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
        const float* vlds = vbuf(t & 1);
#pragma unroll
        for (int cc = 0; cc < G::kCPW; ++cc) {
          const int chunk = G::kKS == 2 ? ks : cc;
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float a = vlds[(chunk * 32 + c_row(i, g)) * G::kVStr + mt * 32 + l32];
              oacc[mt] = mfma_f32(a, pr[cc][i], oacc[mt]);
            }
        }
      }
    }
    // stage V(t+1) and K(t+2), then start loading V(t+2) and K(t+3)
    if (t + 1 < nstage) store_v((t + 1) & 1);
    if (t + 2 < nstage) store_k(t & 1);
    if (t + 2 < nstage) load_v(key0_of(t + 2));
    if (t + 3 < nstage) load_k(key0_of(t + 3));
    __syncthreads();
  };

  f32x16 sa[G::kCPW], sb[G::kCPW];
  if (nstage > 0) {
    load_k(key0_of(0));
    load_v(key0_of(0));
    store_k(0);
    store_v(0);
    if (nstage > 1) load_k(key0_of(1));
    __syncthreads();
    compute_s(0, sa);
    if (nstage > 1) {
      store_k(1);
      load_v(key0_of(1));
    }
    if (nstage > 2) load_k(key0_of(2));
    __syncthreads();
  }
  for (int t = 0; t < nstage; t += 2) {
    step(t, sa, sb);
    if (t + 1 < nstage) step(t + 1, sb, sa);
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
      __syncthreads();  // everyone is done with the stage buffers
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
      float* orow = (float*)p.o + head_off + (size_t)row * D;
#pragma unroll
      for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = mt * 32 + 8 * i4 + 4 * g;
          const float x0 = oacc[mt][4 * i4 + 0] * inv, x1 = oacc[mt][4 * i4 + 1] * inv;
          const float x2 = oacc[mt][4 * i4 + 2] * inv, x3 = oacc[mt][4 * i4 + 3] * inv;
          *(float4*)(orow + d0) = make_float4(x0, x1, x2, x3);
        }
    }
  }
}

// ---------------------------------------------------------------------------
template <int D, int BQ, int MODE>
static hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  using G = Geo<D, BQ, MODE>;
  auto kern = attn_kernel<D, BQ, MODE>;
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t attr = set_lds_limit(kern, G::kLdsBytes, lds_set);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(xcd_grid(p.nb, p.items / p.nb)), dim3(256), G::kLdsBytes, stream, p);
  return hipGetLastError();
}

template <int D, int BQ>
static hipError_t launch_mode(int mode, const AttnParams& p, hipStream_t stream) {
  switch (mode) {
    case kDense: return launch_one<D, BQ, kDense>(p, stream);
    case kSparse: return launch_one<D, BQ, kSparse>(p, stream);
    case kLse: return launch_one<D, BQ, kLse>(p, stream);
    case kMass: return launch_one<D, BQ, kMass>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_fp32(int mode, int head_dim, int block, const AttnParams& p,
                              hipStream_t stream) {
  if (head_dim == 64 && block == 64) return launch_mode<64, 64>(mode, p, stream);
  if (head_dim == 64 && block == 128) return launch_mode<64, 128>(mode, p, stream);
  if (head_dim == 128 && block == 64) return launch_mode<128, 64>(mode, p, stream);
  if (head_dim == 128 && block == 128) return launch_mode<128, 128>(mode, p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn(int mode, int dtype, int head_dim, int block, const AttnParams& p,
                       hipStream_t stream) {
  if (dtype == 0) return launch_attn_bf16(mode, head_dim, block, p, stream);
  if (dtype == 1) return launch_fp32(mode, head_dim, block, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace losa
