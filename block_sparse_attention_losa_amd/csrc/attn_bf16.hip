// bf16 attention passes of the LoSA hot path, written for gfx950 (CDNA4):
//   kDense  - softmax attention over every key block (dense baseline and the
//             construction step's first pass), writes O and lse;
//   kSparse - the same over the frozen key-block list of each query block;
//   kLse    - the row log-sum-exp alone (first pass of the mass map);
//   kMass   - second pass of the mass map: recompute the scores, take
//             exp(s - lse) and sum each (query block, key block) tile;
//   kDenseMass - kDense that also leaves, for every row i and key block J,
//             log2 of the block's share of the row's softmax sum, taken
//             against a per-row reference, in a workspace; once the row's
//             lse is known a small fold turns these into the mass map, so
//             the construction step needs one sweep over the keys, not two.
//
// One workgroup (4 waves) owns 128 query rows -- two 64-row query blocks or
// one 128-row block -- and each wave owns 32 of them; the dense passes at
// D = 128 that write lse use 256-row workgroups of 8 waves (one per CU).  Every 64-key K/V
// tile brought into LDS therefore feeds 128 (or 256) rows, which halves (or
// quarters) the L2 traffic per flop compared with one 64-row block per
// workgroup; at 64 rows the K/V feed alone would need the whole L2
// bandwidth at MFMA peak.  For
// sparse attention the workgroup walks the union of its query blocks' frozen
// lists (ascending) and each wave skips the tiles its own block did not
// keep.  Workgroups take their work item from the XCD-aware default order
// or, for sparse attention, from a launch plan (frozen_lists.hip) that runs
// the items longest-first and evenly over the XCDs.  Q, K, V and O may use
// any bf16 layout with a contiguous head dim (per-tensor element strides).
//
// Data movement is CDNA4-native:
//  * K and V tiles go from HBM straight into LDS with buffer loads in LDS
//    mode (no VGPR staging, no LDS store instructions); rows past the
//    sequence end read as zero through the buffer range check;
//  * tiles are stored row-major with an XOR swizzle of their 16-byte chunks
//    so that both the K fragment reads (ds_read_b128) and the transposing V
//    reads (ds_read_b64_tr_b16, which hand each lane four keys of one head
//    dim) are free of bank conflicts;
//  * in the dense passes with lse, the one-sweep construction at D = 128 and
//    the two passes of the mass map, K runs one tile ahead of V: the scores
//    of tile t+1 are computed on the matrix cores while tile t's softmax
//    runs on the VALU, and the loads of K(t+2) and V(t+1) are in flight
//    during both.  The mass pass and the D = 64 dense pass with lse issue
//    those score MFMAs inside the softmax block, interleaved with the
//    exponentials; the other prefetching 128-row passes issue them ahead of
//    it at a lower wave priority, so the two waves of a SIMD (from different
//    workgroups) tend to alternate between the matrix core and the VALU;
//  * the "lean" passes (lean_pass: sparse attention, dense attention without
//    lse, the one-sweep construction at D = 64) run K and V both one tile
//    ahead and compute a tile's scores in its own step; a wave skips the
//    tiles its block did not keep, and at D = 64 the 32 registers this
//    saves give four waves per SIMD instead of three.  The lean passes
//    without lse take row maxima only on a wave's first kept tile and keep
//    that reference, with a second walk over the tiles for a workgroup
//    whose sums leave the fp32 range.
//
// Scores are computed transposed, S^T = K Q^T, on 32x32x16 MFMA tiles: a
// lane then holds one query row and 16 of the 32 keys of a chunk, so row
// maxima and sums need one cross-half exchange, and the probabilities
// already sit in the B-operand layout of O^T += V^T P^T.  The K rows fed to
// the A operand are permuted (bits 2 and 3 of the row swapped) so that each
// lane's eight probabilities of a 16-key slice are consecutive keys.
#include <type_traits>

#include "attn_common.h"

namespace losa {

template <int D, int BLK, int MODE, int ROWS>
struct GeoB {
  static constexpr bool kWithV = (MODE == kDense || MODE == kSparse || MODE == kDenseMass);
  static constexpr int kRows = ROWS;            // query rows per workgroup (128 or 256)
  static constexpr int kWaves = ROWS / 32;      // one wave per 32 rows
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQPW = kRows / BLK;      // query blocks per workgroup
  static constexpr int kWavesPerBlock = kWaves / kQPW;
  static constexpr int kSubs = BLK / 64;        // 64-key tiles per key block
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTileBytes = 64 * kRowBytes;
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kBlocksPerTile = kTileBytes / 1024;  // 1 KB per wave-wide load
  static constexpr int kBlocksPerWave = kBlocksPerTile / kWaves;
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  static constexpr int kMaxBlocks = 1024;
  static constexpr int kRingBytes = (kWithV ? 4 : 2) * kTileBytes;  // 2 K + 2 V tiles
  static constexpr int kAuxBytes =
      MODE == kSparse ? (2 * kMaxBlocks + 16) * 4 : (MODE == kMass ? 4 * kMaxBlocks * 4 : 0);
  // the last 16 bytes hold the word that sends a workgroup through its
  // tiles a second time (see the tile loop)
  static constexpr int kLdsBytes = kRingBytes + kAuxBytes + 16;
  // sparse: the union list's flags and entries take one slot per key block
  // (rounded up to 64), so a short sequence leaves LDS for more workgroups
  static constexpr int lds_bytes(int nb) {
    return MODE == kSparse ? kRingBytes + (2 * ((nb + 63) / 64) * 64 + 16) * 4 + 16 : kLdsBytes;
  }
};

// "Lean" passes compute a tile's scores at the start of its own step instead
// of one step ahead, and a wave skips outright the tiles its query block did
// not keep.  At D = 64 -- sparse attention, dense attention without lse and
// the one-sweep construction -- this frees the 32
// registers of the second score set and the loop fits 128 VGPRs: four waves
// per SIMD.  A score there carries half the matrix work of D = 128 and the
// same softmax work, so the loop is bound by latency and VALU issue rather
// than the matrix cores, and the fourth wave hides more of it than the
// overlap the score prefetch gave within a wave (sparse, CogVideoX layer:
// 4-5 % faster than three waves with prefetch; one-sweep construction 4 %
// faster; the dense pass with lse keeps the prefetch, which spilled in its
// loop at 128 VGPRs).  At D = 128 the passes without lse (sparse and dense,
// 128-row workgroups) run lean as well, still two waves per SIMD: the
// sparse pass then does no work on the ~3 % of its workgroup's union tiles
// its own query block did not keep, and with the first-tile reference (see
// consume) no per-tile row maxima; measured 3.6-3.7 % faster on the
// Wan2.1-1.3B and HunyuanVideo layers than the prefetching form, and the
// 128-row lean dense pass within 0.3 % of the 256-row prefetching one, so
// sparse attention over every block stays bit-identical to it.  Sparse
// attention with lse (the drift diagnostic) runs lean too, with fp32 row sums
// and the row maxima of every tile: the same arithmetic per tile as the
// dense pass with lse, so bit-identical to it over every block.
constexpr bool lean_pass(int d, int mode, bool mfsum) {
  return mode == kSparse || (mode == kDense && mfsum) || (d == 64 && mode == kDenseMass);
}

// Workgroups per CU the register budget is sized for.  Two waves per SIMD at
// D = 128 (the loop needs ~250 VGPRs); at D = 64 three (168 VGPRs: a third
// wave hides more of the softmax latency than the registers it costs,
// measured 3-4 % faster than two), four for the lean passes.
constexpr int attn_occupancy(int d, int mode, int rows, bool mfsum) {
  return rows == 256 ? 1 : (d == 128 ? 2 : (lean_pass(d, mode, mfsum) ? 4 : 3));
}

template <int D, int BLK, int MODE, int ROWS, bool MFSUM>
__global__ void __launch_bounds__((ROWS * 2), attn_occupancy(D, MODE, ROWS, MFSUM))
    attn_bf16_kernel(AttnParams p) {
  using G = GeoB<D, BLK, MODE, ROWS>;
  static_assert(ROWS == 128 || MODE == kDense || MODE == kDenseMass, "256 rows: dense passes");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int nb = p.nb, N = p.n;
  const int bh_count = p.items / nb;
  const int wph = (nb + G::kQPW - 1) / G::kQPW;  // workgroups per (batch, head)
  // a plan (sparse only) gives the item of each workgroup directly: items
  // ranked by descending cost and assigned to the XCDs in runs of
  // neighbouring query blocks, so every XCD gets the same summed cost and
  // starts with its longest items (layout in frozen_lists.hip); -1 marks an
  // unused slot.  A plan
  // whose header names another shape is not followed: the workgroups then
  // take the items in index order (the grid has a slot for each), so every
  // row is still written
  int item;
  if (p.order != nullptr) {
    const bool match = p.order[0] == kPlanMagic && p.order[1] == wph * bh_count &&
                       p.order[2] == nb && p.order[3] == G::kQPW;
    item = match ? p.order[kPlanHeader + blockIdx.x] : (int)blockIdx.x;
  } else {
    item = xcd_item(blockIdx.x, wph, bh_count);
  }
  // padding of the XCD-aware grid; a plan entry outside the items is ignored
  if (item < 0 || item >= wph * bh_count) return;
  LOSA_POISON(G::kThreads, smem, G::lds_bytes(nb));  // debug build only
  const int bh = item / wph;
  const int w = item - bh * wph;
  const size_t head_off =
      (size_t)(bh / p.heads) * p.stride_b + (size_t)(bh % p.heads) * p.stride_h;
  const int row_stride = (int)p.stride_n * 2;  // bytes between tokens (fits: checked on the host)
  const bf16* __restrict__ qh = (const bf16*)p.q + head_off;
  const bf16* __restrict__ kh = (const bf16*)p.k + head_off;
  const bf16* __restrict__ vh = (const bf16*)p.v + head_off;

  // wave is the same in every lane; saying so once keeps everything derived
  // from it (LDS slot bases of the tile loads, the wave's rows) in scalar
  // registers instead of re-deriving it per use
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int qi = wave / G::kWavesPerBlock;  // this wave's query block within the workgroup
  const int row = w * G::kRows + wave * 32 + l32;
  const bool row_ok = row < N;

  // ---- Q^T as the B operand, in registers (loaded first: the loads overlap
  // the list build below)
  bf16x8 qreg[D / 16];
  {
    // rows past N lie beyond the range and read as zero
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qh, (N - 1) * row_stride + G::kRowBytes);
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk)
      qreg[dk] = __builtin_bit_cast(bf16x8, buf_load16(qr, row * row_stride + dk * 32 + g * 16));
  }

  // ---- key blocks visited, in ascending order, with member bits
  int nblk = nb;
  const int* list = nullptr;
  if constexpr (MODE == kSparse) {
    const int nbpad = ((nb + 63) / 64) * 64;  // as in GeoB::lds_bytes
    int* flag = (int*)(smem + G::kRingBytes);
    int* lst = flag + nbpad;
    int* ccount = lst + nbpad;
    const int qb0 = w * G::kQPW;
    nblk = build_union_list<G::kQPW, G::kThreads, G::kMaxBlocks>(
        p.idx, p.cnt, (size_t)bh * nb + qb0, min(G::kQPW, nb - qb0), nb, flag, lst, ccount);
    list = lst;
  }
  float* part = nullptr;  // kMass: per-wave partial tile sums [4][nb]
  if constexpr (MODE == kMass) {
    part = (float*)(smem + G::kRingBytes);
    for (int j = tid; j < 4 * G::kMaxBlocks; j += 256) part[j] = 0.f;
  }
  auto entry_at = [&](int t) -> int {
    if constexpr (MODE == kSparse) {
      return __builtin_amdgcn_readfirstlane(list[G::kSubs == 1 ? t : (t >> 1)]);
    } else {
      return (G::kSubs == 1 ? t : (t >> 1)) | (((1 << G::kQPW) - 1) << 16);
    }
  };
  int ntile = nblk * G::kSubs;
  if (G::kSubs == 2 && nblk > 0 && (entry_at(ntile - 1) & 0xFFFF) == nb - 1 &&
      (nb - 1) * BLK + 64 >= N)
    --ntile;  // empty second half of a short last block
  auto key0_of = [&](int t) -> int {
    return (entry_at(t) & 0xFFFF) * BLK + (G::kSubs == 1 ? 0 : (t & 1) * 64);
  };

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
    koff[j] = r * row_stride + swz_k<D>(r, pc) * 16;
    voff[j] = r * row_stride + swz_v<D>(r, pc) * 16;
  }
  auto dma_tile = [&](const bf16* src, int key0, unsigned char* slot, const int* off) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc((const unsigned char*)src + (size_t)key0 * row_stride,
                  (N - key0 - 1) * row_stride + G::kRowBytes);
    // wave-uniform LDS destination (M0 must come from a scalar register)
    const unsigned base =
        __builtin_amdgcn_readfirstlane(lds_addr_of(slot) + wave * G::kBlocksPerWave * 1024);
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
  float m_thr = -INFINITY;  // m_run + kRaise: a tile whose scaled max passes it raises m_run
  float m_use = 0.f;        // m_run, or 0 while it is -inf (no finite score yet)
  float l_run = 0.f;        // this lane's partial row sum
  // Row sums on the matrix cores (dense and sparse attention when no lse is
  // asked for): the probabilities are rounded to bf16 for the P V product
  // anyway, and summing exactly those values on a 16x16x32 MFMA takes 32
  // VALU adds per tile off the softmax, the bottleneck at D = 64 (measured
  // 2-3 % faster there, 0.5-1.5 % at D = 128).  O is then normalised by the
  // sum of the very weights it averages V with.  lse needs the unrounded sum
  // (a bf16 probability is off by up to 2^-9 of itself), so when lse is
  // written the adds stay on the VALU in fp32.  The A operand selects, for
  // output row 4*(lane/16), the two lane groups that hold this lane's query
  // row in the B-operand layout of the P V product (lanes q and q + 32), so
  // register 0 of every lane accumulates its own row's full sum.
  constexpr bool kMfmaSum = MFSUM && (MODE == kDense || MODE == kSparse);
  constexpr bool kLean = lean_pass(D, MODE, MFSUM);
  // Lean passes with row sums on the matrix cores keep the reference of a
  // wave's first kept tile (see consume)
  constexpr bool kSpecExp = kLean && kMfmaSum;
  bool spec_first = true;  // kSpecExp: the wave has not yet taken a tile's row maxima
  bool redo = false;       // kSpecExp: second walk over the tiles, exact path on every tile
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  bf16x8 rowsel;
  {
    const int r16 = lane & 15, kg = lane >> 4;
    const bool one = ((r16 == 0 || r16 == 8) && (kg & 1) == 0) ||
                     ((r16 == 4 || r16 == 12) && (kg & 1) == 1);
    const unsigned wv = one ? 0x3F803F80u : 0u;  // bf16 1.0 in both halves
    const u32x4 w4 = {wv, wv, wv, wv};
    rowsel = __builtin_bit_cast(bf16x8, w4);
  }
  const float c2 = p.scale * kLog2e;
  float lse_row = 0.f;      // kMass: the row's lse in log2 units, +inf on padding rows
  float tacc = 0.f;         // kDenseMass: current key block's share of the row sum
  float m0 = 0.f;           // kDenseMass: reference of the first key block
  float pend = 0.f;         // kDenseMass: finished block sum not yet stored ...
  int pend_kb = -1;         // ... and its key block (-1: none)
  auto flush_rowsum = [&]() {
    if constexpr (MODE == kDenseMass) {
      if (pend_kb >= 0) {
        if (g == 0 && row_ok) p.rowsum[((size_t)bh * nb + pend_kb) * N + row] = pend;
        pend_kb = -1;
      }
    }
  };
  // kMass takes exp2(s c log2(e) - lse log2(e)) as one fma and an exp2: the
  // exponent carries the roundings of c log2(e) (times the logit) and of
  // lse log2(e), each <= 2^-24 relative, ~1e-5 for logits near 100 (the
  // softmax that produced lse saw the same c log2(e)); measured 7-8 % faster
  // than fma(s, c, -lse) * log2(e), masses within 7e-7 of it
  if constexpr (MODE == kMass) lse_row = row_ok ? p.lse_in[(size_t)bh * N + row] * kLog2e : INFINITY;

  // S^T of this wave's 32 rows against both 32-key chunks of the K tile
  const int prow = perm_row(l32);
  // At D = 128 the two 32-key chunks' MFMA chains are interleaved, one step
  // of each per head-dim slice, with both chunks' K fragments of a slice read
  // together (measured ~1 % faster there; at D = 64 the chunk-by-chunk order
  // is as fast or faster).  Either way each chunk accumulates its slices in
  // the same order, so the scores are the same bits.
  auto compute_s = [&](const unsigned char* slot, f32x16 (&sc)[2]) {
    if constexpr (D == 128) {
      const int r0 = prow, r1 = 32 + prow;
      const unsigned char* krow0 = slot + r0 * G::kRowBytes;
      const unsigned char* krow1 = slot + r1 * G::kRowBytes;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[0][i] = 0.f;
        sc[1][i] = 0.f;
      }
#pragma unroll
      for (int dk = 0; dk < D / 16; ++dk) {
        const bf16x8 a0 = *(const bf16x8*)(krow0 + swz_k<D>(r0, 2 * dk + g) * 16);
        const bf16x8 a1 = *(const bf16x8*)(krow1 + swz_k<D>(r1, 2 * dk + g) * 16);
        sc[0] = mfma_bf16(a0, qreg[dk], sc[0]);
        sc[1] = mfma_bf16(a1, qreg[dk], sc[1]);
      }
    } else if constexpr (kLean) {
      // the scores are on the step's critical path here: all eight K
      // fragments are read before the first MFMA, so the LDS latency is paid
      // once per tile rather than once per MFMA
      bf16x8 af[2][D / 16];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int r = cc * 32 + prow;
        const unsigned char* krow = slot + r * G::kRowBytes;
#pragma unroll
        for (int dk = 0; dk < D / 16; ++dk)
          af[cc][dk] = *(const bf16x8*)(krow + swz_k<D>(r, 2 * dk + g) * 16);
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[cc][i] = 0.f;
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int dk = 0; dk < D / 16; ++dk) sc[cc] = mfma_bf16(af[cc][dk], qreg[dk], sc[cc]);
    } else {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int r = cc * 32 + prow;
        const unsigned char* krow = slot + r * G::kRowBytes;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[cc][i] = 0.f;
#pragma unroll
        for (int dk = 0; dk < D / 16; ++dk) {
          const bf16x8 a = *(const bf16x8*)(krow + swz_k<D>(r, 2 * dk + g) * 16);
          sc[cc] = mfma_bf16(a, qreg[dk], sc[cc]);
        }
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
    const u32x4 wv = {l2[0], l2[1], h2[0], h2[1]};
    return __builtin_bit_cast(bf16x8, wv);
  };

  // The mass pass (no P V) and the D = 64 dense pass with lse (128-row
  // workgroups) issue the next tile's score MFMAs inside the softmax block
  // (after the rare raise branch), where the scheduler interleaves them with
  // the exponentials: 1-2 % faster than issuing them ahead of it at a lower
  // wave priority, the same bits.  (The 256-row dense passes measured within
  // noise, the D = 64 dense+mass pass 9 % slower.)
  constexpr bool kInline = MODE == kMass || (MODE == kDense && D == 64 && !kLean);

  // keys past the sequence end score -inf (a final tile that runs past N)
  auto mask_tail = [&](f32x16 (&sc)[2], int key0) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + cc * 32 + perm_row(c_row(i, g)) >= N) sc[cc][i] = -INFINITY;
  };
  // bf16 probabilities of tile t against the exponent reference m_e, packed
  // in the B-operand layout of the P V product (slice h of chunk cc)
  auto pack_probs = [&](const f32x16 (&sc)[2], float m_e, u32x4 (&pk)[2][2]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pk[cc][h][j] = pack_bf16x2(
              __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][8 * h + 2 * j], c2, -m_e)),
              __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][8 * h + 2 * j + 1], c2, -m_e)));
  };

  // softmax of tile t (scores in sc) and its P V product; with kInline also
  // the scores of the next tile (K in nslot) into sn
  auto consume = [&](int t, int key0, f32x16 (&sc)[2], auto masked,
                     const unsigned char* nslot, f32x16 (&sn)[2]) {
    if constexpr (decltype(masked)::value) mask_tail(sc, key0);
    if constexpr (MODE == kMass) {
      compute_s(nslot, sn);
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][i], c2, -lse_row));
      acc = wave_sum(acc);
      if (lane == 0) part[wave * G::kMaxBlocks + (key0 / BLK)] += acc;
    } else if constexpr (kSpecExp) {
      // No row maxima after a wave's first kept tile: the probabilities are
      // taken against the reference that tile set, whatever the later
      // scores.  Their bf16 values and the fp32 sums and products keep
      // their relative precision at any size fp32 holds, so the result
      // differs from one taken with a raised reference only in rounding;
      // a row whose later logits exceed its first tile's maximum by more
      // than ~88 (natural units) overflows to inf or NaN, which the check
      // after the tile loop sees, and the workgroup then walks its tiles
      // once more with the lazy rule of the exact path (raise past 2^16)
      // on every tile.  The first kept tile, while the reference is -inf,
      // and every tile of that second walk take the exact path: row
      // maxima, raise and rescale.  Against a test for large probabilities
      // on every tile (packed maxima over the 16 words and a ballot) this
      // drops ~15 VALU instructions per tile.
      if (spec_first || redo) {
        float mx = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[cc][i]);
        mx = pair_max(mx);
        const float m_cand = mx * c2;
        const bool raise = m_cand > m_thr;
        if (__ballot(raise) != 0) {
          float alpha = 1.0f;
          if (raise) {
            alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
            m_run = m_cand;
            m_thr = m_run + kRaise;
            m_use = (m_run == -INFINITY) ? 0.f : m_run;
          }
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mt][i] *= alpha;
          lacc[0] *= alpha;
        }
        spec_first = false;
      }
      u32x4 pk[2][2];
      pack_probs(sc, m_use, pk);
      const unsigned char* vs = vslot[t & 1];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[cc][h]);
          lacc = mfma16_bf16(rowsel, pb, lacc);
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt) {
            const bf16x8 a = v_operand(vs, cc * 32 + h * 16 + g * 8, mt);
            oacc[mt] = mfma_bf16(a, pb, oacc[mt]);
          }
        }
    } else {
      // online softmax; the reference max is raised only when a probability
      // could exceed 2^kRaise, so O is rarely rescaled.  Everything that
      // depends on a raise (the new reference, the rescale factor alpha)
      // lives in a wave-uniform branch taken on those rare tiles; elsewhere
      // alpha is 1, and l + lsum is what fma(l, 1, lsum) rounds to.
      float mx = -INFINITY;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[cc][i]);
      mx = pair_max(mx);
      const float m_cand = mx * c2;
      const bool raise = m_cand > m_thr;
      const bool any_raise = __ballot(raise) != 0;
      float alpha = 1.0f;
      if (any_raise) {
        if (raise) {
          alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
          m_run = m_cand;
          m_thr = m_run + kRaise;
          m_use = (m_run == -INFINITY) ? 0.f : m_run;
        }
        // O is not touched by the exponentials below, so rescaling it here
        // (rather than just before the P V products) gives the same bits,
        // and keeps the whole raise path in one branch
        if constexpr (G::kWithV) {
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mt][i] *= alpha;
        }
        if constexpr (kMfmaSum) lacc[0] *= alpha;
      }
      if constexpr (kInline) compute_s(nslot, sn);
      const float m_e = m_use;
      // with the row sums on the matrix cores the exponentials are taken
      // where the P V product packs them (fewer live registers: at D = 64
      // this removes the loop's spills)
      float pr[2][16];
      float lsum = 0.f;
      if constexpr (!kMfmaSum) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            pr[cc][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][i], c2, -m_e));
            lsum += pr[cc][i];
          }
        // alpha is 1 unless the wave raised, and fma(l, 1, x) rounds exactly
        // like l + x
        l_run = __builtin_fmaf(l_run, alpha, lsum);
      }
      if constexpr (MODE == kDenseMass) {
        // the tile's part of the row sum (both lanes of the row), against
        // the current reference and accumulated over the key block's tiles;
        // after the block's last tile, log2 of it relative to m0 is stored
        // -- at the start of the next step, ahead of that step's tile loads:
        // stores count in vmcnt, and a store issued here would make the
        // end-of-step wait for the loads also wait for its write-back
        const float tsum = pair_sum(lsum);
        tacc = __builtin_fmaf(tacc, alpha, tsum);
        if (G::kSubs == 1 || (key0 % BLK) == BLK - 64 || key0 + 64 >= N) {
          const int kb = key0 / BLK;
          if (kb == 0) m0 = m_run;
          pend = (m_run - m0) + __builtin_amdgcn_logf(tacc);
          pend_kb = kb;
          tacc = 0.f;
        }
      }
      if constexpr (G::kWithV) {
        const unsigned char* vs = vslot[t & 1];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 pk;
            if constexpr (kMfmaSum) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                pk[j] = pack_bf16x2(
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][8 * h + 2 * j], c2, -m_e)),
                    __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cc][8 * h + 2 * j + 1], c2, -m_e)));
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                pk[j] = pack_bf16x2(pr[cc][8 * h + 2 * j], pr[cc][8 * h + 2 * j + 1]);
            }
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
            if constexpr (kMfmaSum) lacc = mfma16_bf16(rowsel, pb, lacc);
#pragma unroll
            for (int mt = 0; mt < kORegs; ++mt) {
              const bf16x8 a = v_operand(vs, cc * 32 + h * 16 + g * 8, mt);
              oacc[mt] = mfma_bf16(a, pb, oacc[mt]);
            }
          }
        }
      }
    }
  };

  // Sparse at D = 128: the list entries of tiles t, t+1 and t+2 as read
  // from LDS (the same value in every lane), carried from step to step.
  // Each step reads the entry of tile t+3, a step before its first use, so
  // the loop never waits on an LDS read of the list (reading entries t, t+1,
  // t+2 where they are used costs one LDS round trip each, per step):
  // measured 1.2 % faster.  At D = 64 the three carried registers spilled
  // (measured with the score prefetch at three waves per SIMD: 2 % slower),
  // so that kernel reads the step's entries together at its start instead,
  // one wait per step (the lean step uses those of tiles t and t+1).
  constexpr bool kWindow = MODE == kSparse && D == 128;
  constexpr bool kBatch = MODE == kSparse && !kWindow;
  int win0 = 0, win1 = 0, win2 = 0;
  auto raw_entry = [&](int t) -> int {
    if constexpr (MODE == kSparse)
      return list[G::kSubs == 1 ? t : (t >> 1)];
    else
      return 0;
  };
  auto key0_from = [&](int e, int t) -> int {
    return (e & 0xFFFF) * BLK + (G::kSubs == 1 ? 0 : (t & 1) * 64);
  };

  // Wave priorities (below) pay off when the waves sharing a SIMD come from
  // different workgroups, whose steps drift apart; in a 256-row
  // workgroup (one per CU) both are in the same workgroup, in lockstep, and
  // equal priorities are 1.3 % faster there.  With kInline the score MFMAs
  // share the softmax block, so there is no separate phase to rank.
  constexpr bool kPrio = ROWS == 128 && !kInline;

  // One pipelined step.  `masked` is true only for a final tile that runs
  // past the sequence end (ascending lists put the short last block last).
  auto step = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2], auto masked) {
    int e0 = 0, e1 = 0, e2 = 0;
    if constexpr (kWindow) {
      e0 = __builtin_amdgcn_readfirstlane(win0);
      e1 = __builtin_amdgcn_readfirstlane(win1);
      e2 = __builtin_amdgcn_readfirstlane(win2);
      win0 = win1;
      win1 = win2;
      // read without a bounds test: past the list it lands in the counts
      // that follow it in LDS, and the value is then never used
      win2 = raw_entry(t + 3);
    } else if constexpr (kBatch) {
      // entries t+1, t+2 are read even past the list (into the counts that
      // follow it in LDS); the loads below use them only when in range
      const int r0 = raw_entry(t);
      const int r1 = raw_entry(t + 1);
      const int r2 = raw_entry(t + 2);
      e0 = __builtin_amdgcn_readfirstlane(r0);
      e1 = __builtin_amdgcn_readfirstlane(r1);
      e2 = __builtin_amdgcn_readfirstlane(r2);
    }
    constexpr bool kHave = kWindow || kBatch;
    const int key0 = kHave ? key0_from(e0, t) : key0_of(t);
    if constexpr (kLean) {
      flush_rowsum();
      // K(t+1) and V(t+1) into the slots tile t-1 freed; then this tile's
      // scores, softmax and P V.  The score MFMAs issue at the lowest wave
      // priority, like the prefetched ones below (0.5-1 % faster than equal
      // priorities here too)
      if (t + 1 < ntile) {
        const int k1 = kHave ? key0_from(e1, t + 1) : key0_of(t + 1);
        LOSA_POISON(G::kThreads, kslot[(t + 1) & 1], G::kTileBytes);  // debug build only
        LOSA_POISON(G::kThreads, vslot[(t + 1) & 1], G::kTileBytes);
        dma_tile(kh, k1, kslot[(t + 1) & 1], koff);
        dma_tile(vh, k1, vslot[(t + 1) & 1], voff);
      }
      if (MODE != kSparse || ((e0 >> (16 + qi)) & 1) != 0) {
        __builtin_amdgcn_s_setprio(0);
        compute_s(kslot[t & 1], sc);
        __builtin_amdgcn_s_setprio(1);
        consume(t, key0, sc, masked, kslot[t & 1], sn);
      }
      wait_dma_all();
      __syncthreads();
      return;
    }
    flush_rowsum();
    // loads for later tiles: K(t+2) into the K slot freed by tile t, V(t+1)
    // into the V slot freed by tile t-1
    if (t + 2 < ntile) {
      LOSA_POISON(G::kThreads, kslot[t & 1], G::kTileBytes);  // debug build only
      dma_tile(kh, kHave ? key0_from(e2, t + 2) : key0_of(t + 2), kslot[t & 1], koff);
    }
    if constexpr (G::kWithV)
      if (t + 1 < ntile) {
        LOSA_POISON(G::kThreads, vslot[(t + 1) & 1], G::kTileBytes);
        dma_tile(vh, kHave ? key0_from(e1, t + 1) : key0_of(t + 1),
                 vslot[(t + 1) & 1], voff);
      }
    // Wave priority (kPrio): the next tile's score MFMAs issue
    // at the lowest level, everything else (softmax, P V, loads, the
    // barrier) one above.  The two waves sharing a SIMD come from different
    // workgroups; when one is in its softmax (the critical path to its P V
    // MFMAs) and the other in its score MFMAs, the softmax issues first and
    // the score MFMAs fill its stalls (measured: 1-3 % faster than equal
    // priorities).
    if constexpr (kInline) {
      consume(t, key0, sc, masked, kslot[(t + 1) & 1], sn);
    } else {
      // scores of the next tile; after the last tile this reads a stale
      // slot and the result is dropped, which keeps the block branch-free
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
      compute_s(kslot[(t + 1) & 1], sn);
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
      consume(t, key0, sc, masked, nullptr, sn);
    }
    wait_dma_all();
    __syncthreads();
  };

  using Plain = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  f32x16 sa[2], sb[2];
  int* redo_word = (int*)(smem + G::lds_bytes(nb) - 16);
  if constexpr (kSpecExp)
    if (tid == 0) *redo_word = 0;  // ordered before any use by the barriers below
  for (;;) {
    LOSA_POISON(G::kThreads, smem, G::kRingBytes);  // debug build only: the tile ring
    if (ntile > 0) {
      dma_tile(kh, key0_of(0), kslot[0], koff);
      if constexpr (G::kWithV) dma_tile(vh, key0_of(0), vslot[0], voff);
      if (!kLean && ntile > 1) dma_tile(kh, key0_of(1), kslot[1], koff);
    }
    // Consume Q (and the row lse) here, on every path: the compiler then waits
    // for those loads once, before the loop, instead of placing vmcnt waits
    // inside the loop where they would also stall on the tile loads in flight.
#pragma unroll
    for (int dk = 0; dk < D / 16; ++dk) asm volatile("" ::"v"(qreg[dk]));
    asm volatile("" ::"v"(lse_row));
    if (ntile > 0) {
      wait_dma_all();
      __syncthreads();
      if (!kLean) {
        compute_s(kslot[0], sa);
        __syncthreads();  // K slot 0 may be refilled from here on
      }
    }
    const bool last_short = ntile > 0 && key0_of(ntile - 1) + 64 > N;
    if constexpr (kWindow) {
      win0 = ntile > 0 ? raw_entry(0) : 0;
      win1 = ntile > 1 ? raw_entry(1) : 0;
      win2 = ntile > 2 ? raw_entry(2) : 0;
    }
    const int nplain = ntile - (last_short ? 1 : 0);
    int t = 0;
    for (; t + 1 < nplain; t += 2) {
      step(t, sa, sb, Plain());
      step(t + 1, sb, sa, Plain());
    }
    if (t < nplain) {
      step(t, sa, sb, Plain());
      ++t;
    }
    if (last_short) {
      if (t & 1)
        step(t, sb, sa, Masked());
      else
        step(t, sa, sb, Masked());
    }

    // kSpecExp: a row sum or output that left the fp32 range (a logit far
    // above the row's first kept tile; see consume) sends the whole
    // workgroup -- the tile loads are shared -- through its tiles again on
    // the exact path.  Finite values pass; inf and NaN do not.
    if constexpr (kSpecExp) {
      if (!redo && ntile > 0) {
        float tot = lacc[0];
#pragma unroll
        for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) tot += fabsf(oacc[mt][i]);
        if (__ballot(!(tot <= 3.0e38f)) != 0 && lane == 0) *redo_word = 1;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(*redo_word) != 0) {
          redo = true;
          spec_first = true;
#pragma unroll
          for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[mt][i] = 0.f;
          lacc = f32x4{0.f, 0.f, 0.f, 0.f};
          m_run = -INFINITY;
          m_thr = -INFINITY;
          m_use = 0.f;
          continue;
        }
      }
    }
    break;
  }

  // ------------------------------------------------------------ epilogue
  if constexpr (MODE == kMass) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < G::kQPW; ++q) {
      const int qb = w * G::kQPW + q;
      if (qb < nb) {
        const float inv_rows = 1.0f / (float)min(BLK, N - qb * BLK);
        float* out = p.mass + ((size_t)bh * nb + qb) * nb;
        const float* pw = part + q * G::kWavesPerBlock * G::kMaxBlocks;
        for (int j = tid; j < nb; j += 256) {
          float tot;
          if constexpr (G::kWavesPerBlock == 4) {
            tot = (pw[j] + pw[G::kMaxBlocks + j]) +
                  (pw[2 * G::kMaxBlocks + j] + pw[3 * G::kMaxBlocks + j]);
          } else {
            tot = pw[j] + pw[G::kMaxBlocks + j];
          }
          out[j] = tot * inv_rows;
        }
      }
    }
    return;
  } else {
    flush_rowsum();
    // (the matrix-core sum already holds both halves of the row)
    const float l_tot = kMfmaSum ? lacc[0] : pair_sum(l_run);
    if (!row_ok) return;
    const bool empty = !(l_tot > 0.f);
    if (p.lse != nullptr && g == 0) {
      p.lse[(size_t)bh * N + row] =
          empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    if constexpr (MODE == kDenseMass) {
      // log2 of the row sum against m0: the fold divides by it
      if (g == 0) p.rowref[(size_t)bh * N + row] = (m_run - m0) + __builtin_amdgcn_logf(l_tot);
    }
    if constexpr (G::kWithV) {
      const float inv = empty ? 0.f : 1.0f / l_tot;
      bf16* orow = (bf16*)p.o + (size_t)(bh / p.heads) * p.o_stride_b +
                   (size_t)(bh % p.heads) * p.o_stride_h + (size_t)row * p.o_stride_n;
#pragma unroll
      for (int mt = 0; mt < kORegs; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = mt * 32 + 8 * i4 + 4 * g;
          u32x2 wv = {pack_bf16x2(oacc[mt][4 * i4 + 0] * inv, oacc[mt][4 * i4 + 1] * inv),
                      pack_bf16x2(oacc[mt][4 * i4 + 2] * inv, oacc[mt][4 * i4 + 3] * inv)};
          *(u32x2*)(orow + d0) = wv;
        }
    }
  }
}

template <int D, int BLK, int MODE, int ROWS = 128, bool MFSUM = false>
hipError_t launch_b(const AttnParams& p, hipStream_t stream) {
  using G = GeoB<D, BLK, MODE, ROWS>;
  auto kern = attn_bf16_kernel<D, BLK, MODE, ROWS, MFSUM>;
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t attr = set_lds_limit(kern, G::kLdsBytes, lds_set);
  if (attr != hipSuccess) return attr;
  const int wph = (p.nb + G::kQPW - 1) / G::kQPW;
  const int grid = p.order != nullptr ? (int)sparse_plan_slots((long long)wph * (p.items / p.nb))
                                       : xcd_grid(wph, p.items / p.nb);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(G::kThreads), G::lds_bytes(p.nb), stream, p);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_b_mode(int mode, const AttnParams& p, hipStream_t stream) {
  switch (mode) {
    // without an lse output the row sums go to the matrix cores
    case kDense:
      return p.lse == nullptr
                 ? launch_b<D, BLK, kDense, attn_rows(kDense, D, BLK, false), true>(p, stream)
                 : launch_b<D, BLK, kDense, attn_rows(kDense, D, BLK)>(p, stream);
    case kSparse:
      return p.lse == nullptr
                 ? launch_b<D, BLK, kSparse, attn_rows(kSparse, D, BLK), true>(p, stream)
                 : launch_b<D, BLK, kSparse, attn_rows(kSparse, D, BLK)>(p, stream);
    case kLse: return launch_b<D, BLK, kLse>(p, stream);
    case kMass: return launch_b<D, BLK, kMass>(p, stream);
    case kDenseMass: return launch_b<D, BLK, kDenseMass, attn_rows(kDenseMass, D, BLK)>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bf16(int mode, int head_dim, int block, const AttnParams& p,
                            hipStream_t stream) {
  if (head_dim == 64 && block == 64) return launch_b_mode<64, 64>(mode, p, stream);
  if (head_dim == 64 && block == 128) return launch_b_mode<64, 128>(mode, p, stream);
  if (head_dim == 128 && block == 64) return launch_b_mode<128, 64>(mode, p, stream);
  if (head_dim == 128 && block == 128) return launch_b_mode<128, 128>(mode, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace losa
