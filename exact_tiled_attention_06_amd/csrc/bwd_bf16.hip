// Backward attention, bf16 storage, on gfx950 MFMA.
//
// Method ("AI基础 | Flash Attention", section 反向传播): the forward kept one
// softmax statistic per row (here the logsumexp LSE); the backward rebuilds
// P = exp(S - LSE) tile by tile from Q, K and the statistic, on chip, and never
// writes an N x N matrix. The gradient formulas are the chain rule on the
// definition:  dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),
// dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Passes (one stream, in order):
//  1. bwd_pre_kernel: per row -D, D = rowsum(dO * O), and -LSE / scale in
//     float32; zeroes the float32 dQ accumulator when dQ is accumulated
//     atomically. The key-block pass starts its S and dP accumulators at these
//     two values, so that the MFMAs hand back S - LSE / scale and dP - D and
//     the softmax rebuild needs one multiply per score less, the dS step one
//     subtraction less.
//  2. bwd_main_kernel: one workgroup per (batch, head, block of 128 keys) —
//     the parallelisation over blocks within one head of the FlashAttention-2
//     paper abstract, item (2), applied to the key axis. Every wavefront owns
//     32 keys and keeps its dK^T and dV^T accumulators in registers while the
//     visible 32-query blocks stream through a 2-stage LDS ring; the block's K
//     stays in LDS (rows padded by 16 bytes in the split pass, swizzled in the
//     atomic one, which also reads it transposed).
//     S = Q K^T and dP = dO V^T are computed with queries on the MFMA rows and
//     the wave's keys on the columns, so P and dS come out of the C registers
//     with eight consecutive queries per lane half: exactly the B operand of
//     dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T are read transposed from
//     LDS with ds_read_b64_tr_b16. dS^T goes through LDS once so that each
//     wave can form a 32 x 32 block of dQ = dS K over all 128 keys of the
//     workgroup, added to the float32 accumulator with global float atomics.
//  3. bwd_dq_convert_kernel: dQ = scale * accumulator, rounded to bf16.
// Deterministic variant: pass 2 skips dQ, and bwd_dq_det_kernel forms dQ per
// 128-query block by a key sweep shaped like the forward (S^T = K Q^T,
// dP^T = V dO^T, dQ^T += K^T dS^T), with no atomics. The full backward runs it
// first, with pass 1 folded in: it holds each query's dO row anyway, so it also
// loads the O row, forms D in pass 1's order of operations and writes both
// per-row values; then pass 2 runs. The separate pass entry points keep pass 1.
// VARLEN (packed sequences of different lengths, deterministic variant only):
// as in the forward, workgroups cover an upper bound of the blocks present and
// find their sequence with varlen_block; D and LSE are [H, total tokens].
// SPARSE (128 x 128 block mask, deterministic variant only): each workgroup
// compacts the tiles of its active blocks into an LDS list and streams only
// those. In the key-block pass a list entry also carries which of the
// workgroup's key blocks are active for that query tile (one at the default
// 128 keys per workgroup, up to two at 256), and a wave whose key block is
// off skips the tile's compute.
// DROPOUT (deterministic variant, fixed-length dense batches): the keep
// matrix of the forward is regenerated from the same Philox4x32-10 counters.
// With Z the keep matrix and r = 1 / (1 - p): dV = (P * Z)^T dO r,
// dS = P * (Z * dP r - D), and D = rowsum(dO * O) is unchanged (O is the
// dropped output). The dQ pass has the forward's query-per-lane layout
// (keep_words_qlane); the key-block pass has one key per lane: each lane
// generates half of one query's 32-key row (keep_rows_klane), the halves merge
// it into 128 bytes of LDS per wave, and each lane reads its key's bits of the
// block's rows from there.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace fa2 {

#ifndef FA2_HEAD_GROUP
#define FA2_HEAD_GROUP 4
#endif
constexpr int kHeadGroup = FA2_HEAD_GROUP;  // heads walked together per XCD

template <int D, int NW_, int NST_, bool DET_>
struct BwdShape {
  static constexpr int NW = NW_;
  static constexpr int NST = NST_;
  static constexpr int NT = NW * 64;
  static constexpr int BK = NW * 32;                    // keys per workgroup
  static constexpr int BQ = 32;                         // queries per iteration
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int KS = D / 16;                     // MFMA steps over d
  static constexpr int MB = D / 32;                     // 32-row blocks of d
  // Resident K tile. The split pass pads its rows by 16 bytes instead of swizzling
  // them (it reads K only along rows); the atomic pass also reads it transposed.
  static constexpr int KROWB = 2 * D + (DET_ ? 16 : 0);
  static constexpr int K_BYTES = BK * KROWB;
  static constexpr int QT_BYTES = BQ * D * 2;           // one Q or dO tile
  static constexpr int STAGE_BYTES = 2 * QT_BYTES + 2 * BQ * 4;
  static constexpr int DS_BYTES = DET_ ? 0 : BK * BQ * 2;  // dS^T, [key][query]
  static constexpr int LDS = K_BYTES + NST * STAGE_BYTES + DS_BYTES;
  // LDS layout: the Q/dO ring first, so that its addresses fit the 16-bit offset
  // field of the LDS instructions, then the resident K tile, then the dS^T tile.
  static constexpr int K_OFF = NST * STAGE_BYTES;
  static_assert(K_OFF % 256 == 0, "K tile offset leaves the row/chunk bits of an address alone");
  static constexpr int DQ_SPLIT = NW / MB;              // waves per d-block in the dQ step
  static constexpr int PER_WAVE = QT_BYTES / (1024 * NW);  // 1 KB direct-load pieces per wave per tile
  static_assert(QT_BYTES % (1024 * NW) == 0, "Q tile must split into 1 KB pieces per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// dS^T tile: rows of 32 queries (64 bytes); chunk c of key row r at c ^ ((r/4)%4).
__device__ __forceinline__ uint32_t ds_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
__device__ __forceinline__ uint32_t ds_off_tr(int r, int col) { return ds_off(r, col >> 3) + (col & 7) * 2; }

// ---------------------------------------------------------------- pass 1
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int zero_acc) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const int64_t total = (int64_t)p.B * p.N * p.H;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;  // token-major (b, i, h)
  const int cc = threadIdx.x % CPR;
  float acc = 0.f;
  if (row < total) {
    const bf16x8 o = *reinterpret_cast<const bf16x8*>((const bf16*)p.o + row * D + cc * 8);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>((const bf16*)p.dout + row * D + cc * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < total) {
    const int64_t h = row % p.H;
    const int64_t i = (row / p.H) % p.N;
    const int64_t b = row / ((int64_t)p.H * p.N);
    const int64_t bhrow = (b * p.H + h) * p.N + i;
    if (cc == 0) {
      if (p.dropout) {
        // The dropout passes rebuild P r, r = 1 / (1 - p), so ln r joins the exponent, and
        // start their dP accumulators at -D / r (the dS step below the key-block pass).
        p.ndelta[bhrow] = -acc * (1.0f / p.drop_scale);
        p.s_init[bhrow] = (logf(p.drop_scale) - p.lse[bhrow]) * p.inv_scale;
      } else {
        p.ndelta[bhrow] = -acc;
        p.s_init[bhrow] = -p.lse[bhrow] * p.inv_scale;
      }
    }
    if (zero_acc) {
      f32x4* dst = reinterpret_cast<f32x4*>(p.dq_acc + bhrow * D + cc * 8);
      dst[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      dst[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// ---------------------------------------------------------------- pass 3
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const int64_t total = (int64_t)p.B * p.N * p.H;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
  const int cc = threadIdx.x % CPR;
  if (row >= total) return;
  const int64_t h = row % p.H;
  const int64_t i = (row / p.H) % p.N;
  const int64_t b = row / ((int64_t)p.H * p.N);
  const int64_t bhrow = (b * p.H + h) * p.N + i;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.dq_acc + bhrow * D + cc * 8);
  const f32x4 x0 = src[0], x1 = src[1];
  const float s = p.scale;
  *reinterpret_cast<bf16x8*>((bf16*)p.dq + row * D + cc * 8) =
      pack_bf16x8(x0[0] * s, x0[1] * s, x0[2] * s, x0[3] * s, x1[0] * s, x1[1] * s, x1[2] * s, x1[3] * s);
}

// ---------------------------------------------------------------- pass 2
// Sequence of this workgroup: head h, first token tok0, length N, and stat0, the
// index of its row 0 in LSE and D. Returns false for a spare workgroup of a
// packed batch. `rows` is the block size of the calling kernel.
template <bool VARLEN>
__device__ __forceinline__ bool bwd_sequence(const BwdParams& p, int rows, bool descending, int& h, int& blk,
                                             int& N, int64_t& tok0, int64_t& stat0) {
  int bh;
  grid_map<kHeadGroup>((int)blockIdx.x, p.nblk, p.B * p.H, descending, bh, blk);
  if constexpr (VARLEN) {
    int t0, len;
    if (!varlen_block(p.cu_seqlens, p.nseq, p.N, rows, blk, blk, t0, len)) return false;
    h = bh;
    N = len;
    tok0 = t0;
    stat0 = (int64_t)h * p.N + t0;
  } else {
    h = bh % p.H;
    N = p.N;
    tok0 = (int64_t)(bh / p.H) * N;
    stat0 = (int64_t)bh * N;
  }
  return true;
}

template <int D, bool ALIBI, bool DET, int NW, int NST, bool VARLEN, bool SPARSE, bool DROPOUT>
__global__ __launch_bounds__(NW * 64, ((D == 128 && !DET) ? 4 : 8) / NW) void bwd_main_kernel(BwdParams p) {
  static_assert(DET || !(VARLEN || SPARSE), "packed and block-sparse batches use the split dQ pass");
  static_assert(!DROPOUT || (DET && !VARLEN && !SPARSE), "dropout: split dQ pass, fixed-length dense batches");
  static_assert(!(VARLEN && SPARSE), "packed batches have no block mask");
  using S = BwdShape<D, NW, NST, DET>;
  static_assert(!SPARSE || (S::BK % kSparseBlock == 0 && S::BK <= 2 * kSparseBlock), "one or two key blocks");
  constexpr int ROWB = 2 * D;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* stage_lds = smem;
  char* k_lds = smem + S::K_OFF;
  char* ds_lds = k_lds + S::K_BYTES;

  int h, kb, N;
  int64_t tok0, stat0;
  if (!bwd_sequence<VARLEN>(p, S::BK, false, h, kb, N, tok0, stat0)) return;  // early keys first
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, j = lane & 15;
  const int64_t rs = (int64_t)p.H * D;
  const int64_t base = tok0 * rs + (int64_t)h * D;
  const bf16* qg = (const bf16*)p.q + base;
  const bf16* kg = (const bf16*)p.k + base;
  const bf16* vg = (const bf16*)p.v + base;
  const bf16* dog = (const bf16*)p.dout + base;
  const float* sinit_g = p.s_init + stat0;  // -LSE / scale
  const float* ndel_g = p.ndelta + stat0;   // -D

  const int k0 = kb * S::BK;
  const int k_last = min(k0 + S::BK, N) - 1;
  const int kw0 = k0 + 32 * w;  // first key of this wave
  const int kj = kw0 + l32;     // key of this lane (MFMA column)
  const int bh = (int)(stat0 / (N > 0 ? N : 1));            // b * H + h (fixed-length batches)
  uint32_t* drop_slot = reinterpret_cast<uint32_t*>(smem + S::LDS) + 32 * w;  // DROPOUT: 32 words per wave
  const int drop_pos = keep_row_bit(l32);  // DROPOUT: this lane's key in a row mask

  // V^T fragments (B operand of dP = dO V^T): lane holds v[kj][16*ks + 8*hh .. +7].
  bf16x8 vf[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks)
    vf[ks] = kj < N ? *reinterpret_cast<const bf16x8*>(vg + (int64_t)kj * rs + 16 * ks + 8 * hh) : bf16x8{};
  // Resident K tile (B operand of S, and K of dQ = dS K). Split pass: padded rows
  // (pitch 2d + 16 bytes), so that the reads of the d-steps differ by constant
  // offsets and the 16-byte shift per row spreads one column over all banks; rows
  // past the sequence repeat its last row.
  constexpr int K_PER_T = S::BK * S::CPR / S::NT;  // 16-byte pieces per thread
  bf16x8 kpiece[DET ? K_PER_T : 1];
  if constexpr (DET) {
#pragma unroll
    for (int n = 0; n < K_PER_T; ++n) {
      const int c = tid + n * S::NT, row = c / S::CPR;
      const int key = min(k0 + row, N - 1);
      kpiece[n] = *reinterpret_cast<const bf16x8*>(kg + (int64_t)key * rs + (c % S::CPR) * 8);
    }
  }
  wait_vm_all();
  if constexpr (DET) {
#pragma unroll
    for (int n = 0; n < K_PER_T; ++n) {
      const int c = tid + n * S::NT;
      *reinterpret_cast<bf16x8*>(k_lds + (c / S::CPR) * S::KROWB + (c % S::CPR) * 16) = kpiece[n];
    }
  } else {
    dma_tile<D, S::BK, NW>(k_lds, kg, rs, k0, N, w, lane);
  }

  const float slope2 = ALIBI ? p.alibi[h] * kLog2e : 0.f;

  // Query blocks that can see any key of this workgroup.
  int q_lo = 0, q_hi = N - 1;
  if (p.wr >= 0) q_lo = max(0, k0 - p.wr);
  if (p.wl >= 0) q_hi = min(N - 1, k_last + p.wl);
  const int it_lo = q_lo / S::BQ, it_hi = q_hi / S::BQ + 1;

  // The query tiles to visit: it_lo .. it_hi - 1, or for SPARSE those of active
  // blocks, each with a bit per key block of this workgroup (bit 0: keys k0 ..
  // k0 + 127, bit 1: the next 128).
  uint16_t* tile_list = reinterpret_cast<uint16_t*>(smem + S::LDS);
  int n_tiles = it_hi - it_lo;
  if constexpr (SPARSE) {
    const uint8_t* mbh = p.block_mask + (tok0 / N) * p.mask_sb + (int64_t)h * p.mask_sh;
    const int c0 = k0 / kSparseBlock;
    const bool two = S::BK > kSparseBlock && c0 + 1 < p.nbk;
    static_assert(kSparseBlock % S::BQ == 0, "whole query tiles per mask block");
    n_tiles = compact_tiles(tile_list, it_lo, it_hi, kSparseBlock / S::BQ, w, [&](int r) -> uint32_t {
      const uint8_t* row = mbh + (int64_t)r * p.nbk + c0;  // mask row r: query block r
      return (row[0] != 0 ? 1u : 0u) | (two && row[1] != 0 ? 2u : 0u);
    });
    __syncthreads();
  }
  auto entry_at = [&](int u) __attribute__((always_inline)) -> uint32_t {
    if constexpr (SPARSE) {
      return __builtin_amdgcn_readfirstlane((uint32_t)tile_list[u]);
    } else {
      return (uint32_t)(it_lo + u);
    }
  };

  // Per-lane LDS bases; every read below is base ^ constant or base + constant.
  const int ar = kperm(l32);  // A-operand row (query) for S and dP
  uint32_t qa_base = ar * ROWB + ((hh ^ tile_swz<D>(ar)) << 4);
  // Its addresses for the d-steps, kept in registers across the loop (formed per
  // block instead under dropout, whose generator needs the registers).
  constexpr bool KEEP_QX = !DROPOUT;
  uint32_t qx[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) {
    qx[ks] = qa_base ^ (ks << 5);
    if (KEEP_QX) opaque(qx[ks]);
  }
  // K rows of this wave's keys, as LDS addresses: padded rows (split pass), or
  // swizzled ones (K_OFF is a multiple of 256, so XOR with a chunk offset below 256
  // commutes with adding it).
  uint32_t kb_base = DET ? S::K_OFF + (32 * w + l32) * S::KROWB + (hh << 4)
                         : S::K_OFF + (32 * w + l32) * ROWB + ((hh ^ tile_swz<D>(l32)) << 4);
  const int tr0 = 8 * hh + (j >> 2);
  const int c0 = 2 * (g & 1) + ((j & 3) >> 1);
  uint32_t tr_lo = tr0 * ROWB + ((c0 ^ tile_swz<D>(tr0)) << 4) + (j & 1) * 8;
  uint32_t tr_hi = (tr0 + 4) * ROWB + ((c0 ^ tile_swz<D>(tr0 + 4)) << 4) + (j & 1) * 8;
  // dQ step: dS^T rows / K rows part*KSPAN + 8*hh + j/4 (+4) (+16*kk).
  const int mbq = w % S::MB, part = w / S::MB;
  constexpr int KSPAN = S::BK / S::DQ_SPLIT;
  const int dr0 = part * KSPAN + tr0;
  uint32_t ds_lo = dr0 * 64 + ((c0 ^ ((dr0 >> 2) & 3)) << 4) + (j & 1) * 8;
  uint32_t ds_hi = (dr0 + 4) * 64 + ((c0 ^ (((dr0 + 4) >> 2) & 3)) << 4) + (j & 1) * 8;
  const int kc0 = 4 * mbq + c0;  // K chunk for the dQ B operand
  uint32_t kt_lo = dr0 * ROWB + ((kc0 ^ tile_swz<D>(dr0)) << 4) + (j & 1) * 8;
  uint32_t kt_hi = (dr0 + 4) * ROWB + ((kc0 ^ tile_swz<D>(dr0 + 4)) << 4) + (j & 1) * 8;

  f32x16 dk[S::MB], dv[S::MB];
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) {
    dk[mb] = f32x16{};
    dv[mb] = f32x16{};
  }

  // Per-lane byte offsets of this lane's direct-load pieces of a Q/dO tile.
  constexpr int PER_WAVE = S::PER_WAVE;
  uint32_t dma_off[PER_WAVE];
#pragma unroll
  for (int n = 0; n < PER_WAVE; ++n) {
    const int byte = (w * PER_WAVE + n) * 1024 + 16 * lane;
    const int r = byte / ROWB;
    const int cc = ((byte % ROWB) >> 4) ^ tile_swz<D>(r);
    dma_off[n] = (uint32_t)(r * rs * 2 + cc * 16);
  }

  // Q, dO (swizzled tiles) and LSE, D (raw floats) of query block `it` into a stage.
  auto issue_q = [&](int it, auto stage_c) __attribute__((always_inline)) {
    constexpr int stg = decltype(stage_c)::value;
    char* st = stage_lds + stg * S::STAGE_BYTES;
    const int i0 = it * S::BQ;
    if (i0 + S::BQ <= N) {
      const char* qgb = reinterpret_cast<const char*>(qg + (int64_t)i0 * rs);
      const char* ogb = reinterpret_cast<const char*>(dog + (int64_t)i0 * rs);
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        char* dst = st + (w * PER_WAVE + n) * 1024;
        dma16(qgb, dma_off[n], dst);
        dma16(ogb, dma_off[n], dst + S::QT_BYTES);
      }
    } else {  // last, partial block: clamp rows to the sequence
      dma_tile<D, S::BQ, S::NW>(st, qg, rs, i0, N, w, lane);
      dma_tile<D, S::BQ, S::NW>(st + S::QT_BYTES, dog, rs, i0, N, w, lane);
    }
    if (w == 0) {
      const int q = min(i0 + l32, N - 1);
      const float* src = hh ? ndel_g + q : sinit_g + q;
      dma4(src, st + 2 * S::QT_BYTES);
    }
  };

  // Waits until the next query block has landed; `younger` blocks issued after
  // it may stay in flight (wave 0 issues one extra load per block, for LSE and D).
  auto wait_next = [&](int younger) __attribute__((always_inline)) {
    if (w == 0) {
      wait_ring<NST, 2 * PER_WAVE + 1>(younger);
    } else {
      wait_ring<NST, 2 * PER_WAVE>(younger);
    }
  };

  // One 32-query block (the u-th to visit); the stage is a compile-time constant.
  auto body = [&](int u, auto stage_c) __attribute__((always_inline)) {
    constexpr int stg = decltype(stage_c)::value;
    if (u + NST - 1 < n_tiles)
      issue_q((int)(entry_at(u + NST - 1) & kTileIndexMask), std::integral_constant<int, (stg + NST - 1) % NST>{});
    if (!KEEP_QX) {
      opaque(qa_base);
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) qx[ks] = qa_base ^ (ks << 5);
    }
    opaque(kb_base);
    opaque(tr_lo);
    opaque(tr_hi);
    const uint32_t ent = entry_at(u);
    const int it = (int)(ent & kTileIndexMask);
    const int i0 = it * S::BQ;
    const int i1 = i0 + S::BQ - 1;
    // SPARSE: this wave's key block (32 keys per wave, 128 per block) must be active
    const bool off = SPARSE && ((ent >> 14) & (1u << ((32 * w) / kSparseBlock))) == 0;
    const bool skip = off || kw0 >= N || (p.wr >= 0 && i1 + p.wr < kw0) || (p.wl >= 0 && i0 - p.wl > kw0 + 31);
    if (!skip) {
      // LDS addresses (the dynamic buffer starts at 0: the launcher checks there is no
      // static LDS): this stage's Q and dO tiles; the K tile sits at K_OFF.
      constexpr uint32_t kQ = stg * S::STAGE_BYTES, kDO = kQ + S::QT_BYTES;
      const char* q_t = stage_lds + stg * S::STAGE_BYTES;
      const float* sinit_t = reinterpret_cast<const float*>(q_t + 2 * S::QT_BYTES);  // -LSE / scale
      const float* ndel_t = sinit_t + S::BQ;                                           // -D

      // S - LSE / scale = Q K^T - LSE / scale: rows are queries (A lane m reads row
      // kperm(m)), columns are this wave's keys; register r holds query key_of_reg(r, hh).
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = sinit_t[key_of_reg(r, hh)];
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        const bf16x8 a = lds_read16_at(kQ + qx[ks]);
        const bf16x8 bk = lds_read16_at(DET ? kb_base + (ks << 5) : kb_base ^ (ks << 5));
        s = mfma32(a, bk, s);
      }
      // Masks. Dense and packed batches mask S in place (-inf for hidden keys), a branch
      // that rewrites S where it lies; every row there has a finite LSE. Block-sparse
      // batches can have rows without a visible key (LSE = -inf) and mask P instead.
      const bool full = i1 < N && kw0 + 31 < N && (p.wr < 0 || i0 + p.wr >= kw0 + 31) &&
                        (p.wl < 0 || i1 - p.wl <= kw0);
      auto visible = [&](int r) __attribute__((always_inline)) {
        const int q = i0 + key_of_reg(r, hh);
        return q < N && kj < N && (p.wr < 0 || kj <= q + p.wr) && (p.wl < 0 || kj >= q - p.wl);
      };
      if (!SPARSE && !full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = visible(r) ? s[r] : -INFINITY;
      }
      // P = exp2((S - LSE / scale) * scale * log2e + bias), bias = -slope * |i - j|.
      float y[16];
      if (ALIBI && (kw0 + 31 <= i0 || kw0 >= i1)) {
        // Every key of the wave on one side of every query of the tile: |i - j| = +-(i - j)
        // and i - j = (i0 + 8 hh - kj) + key_of_reg(r, 0), a constant per register.
        const float ss = kw0 + 31 <= i0 ? -slope2 : slope2;  // bias = ss * (i - j)
        const float b0 = ss * (float)(i0 + 8 * hh - kj);
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = fmaf(s[r], p.scale_log2, fmaf(ss, (float)key_of_reg(r, 0), b0));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          y[r] = s[r] * p.scale_log2;
          if (ALIBI) y[r] = fmaf(-slope2, fabsf((float)(i0 + key_of_reg(r, hh) - kj)), y[r]);
        }
      }
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(y[r]);
      if (SPARSE && !full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = visible(r) ? pr[r] : 0.f;
      }
      // Keep bits (dropout) between the two products: S is dead and dP not yet live.
      // One generator call per lane and block: the rows of the block's queries go into
      // the wave's slot, and each lane reads the bits of its key from there.
      const uint32_t* keep_rows = drop_slot;
      if constexpr (DROPOUT) {
        keep_rows_klane(p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_keep, bh, i0, kw0, l32, hh, drop_slot);
        keep_rows = drop_slot + 8 * hh;
      }
      // dP - D = dO V^T - D, then dS = P * (dP - D) (under dropout the accumulators start
      // at 0 and dS = P * (Z * dP / (1 - p) - D)).
      f32x16 dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = ndel_t[key_of_reg(r, hh)];
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        const bf16x8 ao = lds_read16_at(kDO + qx[ks]);
        dp = mfma32(ao, vf[ks], dp);
      }
      // Under dropout pr holds P r and dp holds dP - D / r, so dS = P (Z dP r - D) is
      // pr * dp where Z keeps and pr * (-D / r) where it drops; dV takes Z P r. The
      // -D / r values are read again here, so that they hold no registers across the MFMAs.
      float nd[16];
      if constexpr (DROPOUT) {
        uint32_t nd_addr = kQ + 2 * S::QT_BYTES + S::BQ * 4 + 32 * hh;  // ndel_t + 8 hh
        opaque(nd_addr);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 x = lds_read_f32x4_at(nd_addr + 16 * (c & 1) + 64 * (c >> 1));  // registers 4c .. 4c+3
#pragma unroll
          for (int e = 0; e < 4; ++e) nd[4 * c + e] = x[e];
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float d8[8], pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * kk + e;
          if constexpr (DROPOUT) {
            const uint32_t z = keep_mask_of(drop_row(keep_rows, r), drop_pos);  // all ones: kept
            d8[e] = pr[r] * select_bits(z, dp[r], nd[r]);
            pk[e] = select_bits(z, pr[r], 0.f);
          } else {
            d8[e] = pr[r] * dp[r];
            pk[e] = pr[r];
          }
        }
        pb[kk] = pack_bf16x8(pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]);
        dsb[kk] = pack_bf16x8(d8[0], d8[1], d8[2], d8[3], d8[4], d8[5], d8[6], d8[7]);
      }
      if (!DET) {
        const int row = 32 * w + l32;  // key row of dS^T; chunk c holds queries 8c .. 8c+7
        *reinterpret_cast<bf16x8*>(ds_lds + ds_off(row, hh)) = dsb[0];
        *reinterpret_cast<bf16x8*>(ds_lds + ds_off(row, 2 + hh)) = dsb[1];
      }
      // dV^T += dO^T P and dK^T += Q^T dS (A operands read transposed from LDS).
      uint32_t tx_lo[S::MB], tx_hi[S::MB];
#pragma unroll
      for (int mb = 0; mb < S::MB; ++mb) {
        tx_lo[mb] = tr_lo ^ (mb << 6);
        tx_hi[mb] = tr_hi ^ (mb << 6);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int mb = 0; mb < S::MB; ++mb) {
          const int ro = kk * 16 * ROWB;
          const bf16x4 o_lo = lds_read_tr_at(kDO + ro + tx_lo[mb]);
          const bf16x4 o_hi = lds_read_tr_at(kDO + ro + tx_hi[mb]);
          dv[mb] = mfma32(__builtin_shufflevector(o_lo, o_hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[kk], dv[mb]);
          const bf16x4 q_lo = lds_read_tr_at(kQ + ro + tx_lo[mb]);
          const bf16x4 q_hi = lds_read_tr_at(kQ + ro + tx_hi[mb]);
          dk[mb] = mfma32(__builtin_shufflevector(q_lo, q_hi, 0, 1, 2, 3, 4, 5, 6, 7), dsb[kk], dk[mb]);
        }
      }
    } else if (!DET) {
      const int row = 32 * w + l32;
      *reinterpret_cast<u32x4*>(ds_lds + ds_off(row, hh)) = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(ds_lds + ds_off(row, 2 + hh)) = u32x4{0, 0, 0, 0};
    }
    if (!DET) {
      __syncthreads();  // dS^T of all waves is in LDS
      opaque(ds_lo);
      opaque(ds_hi);
      opaque(kt_lo);
      opaque(kt_hi);
      // dQ block: rows i0..i0+31, d columns 32*mbq .. +31, over this wave's share of the keys.
      f32x16 dqa = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KSPAN / 16; ++kk) {
        const bf16x4 a_lo = lds_read_tr(ds_lds + ds_lo + kk * 16 * 64);
        const bf16x4 a_hi = lds_read_tr(ds_lds + ds_hi + kk * 16 * 64);
        const bf16x4 b_lo = lds_read_tr(k_lds + kt_lo + kk * 16 * ROWB);
        const bf16x4 b_hi = lds_read_tr(k_lds + kt_hi + kk * 16 * ROWB);
        dqa = mfma32(__builtin_shufflevector(a_lo, a_hi, 0, 1, 2, 3, 4, 5, 6, 7),
                     __builtin_shufflevector(b_lo, b_hi, 0, 1, 2, 3, 4, 5, 6, 7), dqa);
      }
      float* dq_row = p.dq_acc + (stat0 + i0) * D + 32 * mbq + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r >> 2) + 4 * hh + (r & 3);
        if (i0 + m < N) atomicAdd(dq_row + (int64_t)m * D, dqa[r]);
      }
    }
    wait_next(n_tiles - u - 2);  // block u + 1
  };

  static_for<0, NST - 1>([&](auto sc) {
    constexpr int k = decltype(sc)::value;
    if (k < n_tiles) issue_q((int)(entry_at(k) & kTileIndexMask), std::integral_constant<int, k>{});
  });
  wait_next(n_tiles - 1);  // block 0
  for (int u = 0; u < n_tiles; u += NST) {
    static_for<0, NST>([&](auto sc) {
      constexpr int k = decltype(sc)::value;
      if (u + k < n_tiles) body(u + k, sc);
    });
  }

  // dK = scale * dK^T, dV = dV^T, stored as bf16: lane holds key kj, d = 32*mb + 8*a + 4*hh + (0..3).
  if (kj < N) {
    bf16* dk_row = (bf16*)p.dk + base + (int64_t)kj * rs;
    bf16* dv_row = (bf16*)p.dv + base + (int64_t)kj * rs;
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 xk, xv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xk[e] = (bf16)(dk[mb][4 * a + e] * p.scale);
          xv[e] = (bf16)dv[mb][4 * a + e];
        }
        *reinterpret_cast<bf16x4*>(dk_row + 32 * mb + 8 * a + 4 * hh) = xk;
        *reinterpret_cast<bf16x4*>(dv_row + 32 * mb + 8 * a + 4 * hh) = xv;
      }
    }
  }
}

// ---------------------------------------------------------------- deterministic dQ
// One workgroup per (batch, head, 128-query block); every wave owns 32 query
// rows and sweeps the visible 32-key tiles like the forward: S^T = K Q^T and
// dP^T = V dO^T put one query per lane (column), so LSE and D are per-lane
// scalars, and dS^T feeds dQ^T += K^T dS^T as the B operand straight from
// registers (K^T read transposed from the K tile).
template <int D, bool ALIBI, int NW, int NST, bool VARLEN, bool SPARSE, bool DROPOUT>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_det_kernel(BwdParams p) {  // 2 waves per SIMD
  static_assert(!(VARLEN && SPARSE), "packed batches have no block mask");
  static_assert(!DROPOUT || !(VARLEN || SPARSE), "dropout runs on fixed-length dense batches");
  static_assert(!SPARSE || NW * 32 == kSparseBlock, "a workgroup covers one mask row");
  constexpr int BR = NW * 32, BC = 32;
  constexpr int KS = D / 16, MB = D / 32;
  constexpr int ROWB = 2 * D;
  constexpr int TILE = BC * D * 2;
  constexpr int STAGE = 2 * TILE;
  constexpr int PER_WAVE = TILE / (1024 * NW);
  static_assert(TILE % (1024 * NW) == 0, "tile must split into 1 KB pieces per wave");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  int h, qb, N;
  int64_t tok0, stat0;
  if (!bwd_sequence<VARLEN>(p, BR, true, h, qb, N, tok0, stat0)) return;  // longest blocks first
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, j = lane & 15;
  const int64_t rs = (int64_t)p.H * D;
  const int64_t base = tok0 * rs + (int64_t)h * D;
  const bf16* qg = (const bf16*)p.q + base;
  const bf16* kg = (const bf16*)p.k + base;
  const bf16* vg = (const bf16*)p.v + base;
  const bf16* dog = (const bf16*)p.dout + base;

  const int q0 = qb * BR;
  const int q_last = min(q0 + BR, N) - 1;
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + l32;
  const bool wave_live = qw0 < N;
  const int wq_last = min(qw0 + 31, N - 1);
  const int bh = (int)(stat0 / (N > 0 ? N : 1));  // b * H + h (fixed-length batches)

  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = qi < N ? *reinterpret_cast<const bf16x8*>(qg + (int64_t)qi * rs + 16 * ks + 8 * hh) : bf16x8{};
    of[ks] = qi < N ? *reinterpret_cast<const bf16x8*>(dog + (int64_t)qi * rs + 16 * ks + 8 * hh) : bf16x8{};
  }
  // +inf for rows past the end and for rows without a visible key (LSE = -inf): their
  // masked scores (-inf) then give P = exp2(-inf - lse2) = 0 without a NaN.
  const float lse_qi = qi < N ? p.lse[stat0 + qi] : -INFINITY;
  // Under dropout the pass rebuilds P r, r = 1 / (1 - p): log2 r comes off the statistic.
  const float lse2 = lse_qi > -INFINITY ? lse_qi * kLog2e - (DROPOUT ? log2f(p.drop_scale) : 0.f) : INFINITY;
  float ndelta;  // -D (-D / r under dropout)
  if (p.fuse_stats) {
    // D = rowsum(dO * O) of this lane's query, and the two per-row values the key-block
    // pass reads, in bwd_pre_kernel's order of operations so that they are bit for bit
    // its values: an 8-element dot product per 16-byte chunk (chunk 2 ks + hh here),
    // then sums of chunks c and c ^ off for off = d / 16 .. 1 (the last across halves).
    const bf16* og = (const bf16*)p.o + base;
    float part[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 o8 = qi < N ? *reinterpret_cast<const bf16x8*>(og + (int64_t)qi * rs + 16 * ks + 8 * hh) : bf16x8{};
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o8[e], (float)of[ks][e], acc);
      part[ks] = acc;
    }
#pragma unroll
    for (int half = KS / 2; half >= 1; half >>= 1) {
#pragma unroll
      for (int ks = 0; ks < half; ++ks) part[ks] += part[ks + half];
    }
    const float dsum = part[0] + __uint_as_float(from_other_half(__float_as_uint(part[0])));
    ndelta = p.dropout ? -dsum * (1.0f / p.drop_scale) : -dsum;
    if (hh == 0 && qi < N) {
      p.ndelta[stat0 + qi] = ndelta;
      p.s_init[stat0 + qi] = p.dropout ? (logf(p.drop_scale) - lse_qi) * p.inv_scale : -lse_qi * p.inv_scale;
    }
  } else {
    ndelta = qi < N ? p.ndelta[stat0 + qi] : 0.f;
  }
  // dP^T accumulators start at ndelta (every register of a lane holds this lane's query),
  // so that the MFMAs hand back dP - D (dP - D / r).
  f32x16 dp_init;
#pragma unroll
  for (int r = 0; r < 16; ++r) dp_init[r] = ndelta;
  const float slope2 = ALIBI ? p.alibi[h] * kLog2e : 0.f;

  int kv_lo = 0, kv_hi = N;
  if (p.wl >= 0) kv_lo = max(0, q0 - p.wl);
  if (p.wr >= 0) kv_hi = min(N, q_last + p.wr + 1);
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;

  // The key tiles to visit: t_lo .. t_hi - 1, or for SPARSE those of active key blocks.
  uint16_t* tile_list = reinterpret_cast<uint16_t*>(smem + NST * STAGE);
  int n_tiles = t_hi - t_lo;
  if constexpr (SPARSE) {
    const uint8_t* mrow = p.block_mask + (tok0 / N) * p.mask_sb + (int64_t)h * p.mask_sh + (int64_t)qb * p.nbk;
    static_assert(kSparseBlock % BC == 0, "whole tiles per mask block");
    n_tiles = compact_tiles(tile_list, t_lo, t_hi, kSparseBlock / BC, w,
                            [&](int b) -> uint32_t { return mrow[b] != 0 ? 1u : 0u; });
    __syncthreads();
  }
  // Key tiles from the last down: with the longest blocks started first, a
  // workgroup that starts when another ends reads tiles its running neighbours
  // read shortly before (for this pass it missed L2 less than ascending).
  auto tile_at = [&](int u) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) {
      return __builtin_amdgcn_readfirstlane((int)(tile_list[n_tiles - 1 - u] & kTileIndexMask));
    } else {
      return t_hi - 1 - u;
    }
  };

  uint32_t dma_off[PER_WAVE];
#pragma unroll
  for (int n = 0; n < PER_WAVE; ++n) {
    const int byte = (w * PER_WAVE + n) * 1024 + 16 * lane;
    const int r = byte / ROWB;
    const int cc = ((byte % ROWB) >> 4) ^ tile_swz<D>(r);
    dma_off[n] = (uint32_t)(r * rs * 2 + cc * 16);
  }
  const int kr = kperm(l32);
  uint32_t abase = kr * ROWB + ((hh ^ tile_swz<D>(kr)) << 4);  // K, V rows (A operands)
  // Its addresses for the d-steps, kept in registers across the loop (formed per
  // tile instead under dropout, whose generator needs the registers).
  constexpr bool KEEP_AX = !DROPOUT;
  uint32_t ax[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    ax[ks] = abase ^ (ks << 5);
    if (KEEP_AX) opaque(ax[ks]);
  }
  const int tr0 = 8 * hh + (j >> 2);
  const int c0 = 2 * (g & 1) + ((j & 3) >> 1);
  uint32_t tr_lo = tr0 * ROWB + ((c0 ^ tile_swz<D>(tr0)) << 4) + (j & 1) * 8;
  uint32_t tr_hi = (tr0 + 4) * ROWB + ((c0 ^ tile_swz<D>(tr0 + 4)) << 4) + (j & 1) * 8;

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};

  auto issue = [&](int t, auto stage_c) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_c)::value;
    char* kl = smem + st * STAGE;
    const int row0 = t * BC;
    if (row0 + BC <= N) {
      const char* kgb = reinterpret_cast<const char*>(kg + (int64_t)row0 * rs);
      const char* vgb = reinterpret_cast<const char*>(vg + (int64_t)row0 * rs);
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        char* dst = kl + (w * PER_WAVE + n) * 1024;
        dma16(kgb, dma_off[n], dst);
        dma16(vgb, dma_off[n], dst + TILE);
      }
    } else {
      dma_tile<D, BC, NW>(kl, kg, rs, row0, N, w, lane);
      dma_tile<D, BC, NW>(kl + TILE, vg, rs, row0, N, w, lane);
    }
  };

  auto body = [&](int u, auto stage_c) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_c)::value;
    if (u + NST - 1 < n_tiles) issue(tile_at(u + NST - 1), std::integral_constant<int, (st + NST - 1) % NST>{});
    const int t = tile_at(u);
    if (!KEEP_AX) {
      opaque(abase);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ax[ks] = abase ^ (ks << 5);
    }
    opaque(tr_lo);
    opaque(tr_hi);
    const int j0 = t * BC, j1 = j0 + BC - 1;
    const bool skip = !wave_live || (p.wr >= 0 && j0 > wq_last + p.wr) || (p.wl >= 0 && j1 < qw0 - p.wl);
    if (!skip) {
      // LDS addresses of this stage's K and V tiles (the dynamic buffer starts at 0:
      // the launcher checks there is no static LDS).
      constexpr uint32_t kK = st * STAGE, kV = kK + TILE;
      // S^T = K Q^T and dP^T = V dO^T: rows are keys (A lane m reads row kperm(m)), columns queries.
      // The K and V fragments of step ks + 1 are read while the MFMAs of step ks run.
      f32x16 s = f32x16{}, dp = dp_init;
      if constexpr (DROPOUT) {
        // Formed per tile: a 16-register copy held across the loop would cost the
        // generator's registers.
        float nd = ndelta;
        opaque(nd);
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = nd;
      }
      bf16x8 kv[2][2];
      auto kvload = [&](int ks, bf16x8(&dst)[2]) __attribute__((always_inline)) {
        dst[0] = lds_read16_at(kK + ax[ks]);
        dst[1] = lds_read16_at(kV + ax[ks]);
      };
      kvload(0, kv[0]);
      static_for<0, KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 1 < KS) kvload(ks + 1, kv[(ks + 1) & 1]);
        s = mfma32(kv[ks & 1][0], qf[ks], s);
        dp = mfma32(kv[ks & 1][1], of[ks], dp);
      });
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS reads of steps 0 and 1
      static_for<0, KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, ks + 1 < KS ? 2 : 0, 0);  // reads of step ks + 2
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                    // MFMAs of step ks
      });
      // K^T fragments for dQ^T += K^T dS^T (both 16-key halves), read ahead of the softmax.
      uint32_t tx_lo[MB], tx_hi[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        tx_lo[mb] = tr_lo ^ (mb << 6);
        tx_hi[mb] = tr_hi ^ (mb << 6);
      }
      bf16x8 kt[2][MB];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ro = kk * 16 * ROWB;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x4 lo = lds_read_tr_at(kK + ro + tx_lo[mb]);
          const bf16x4 hi = lds_read_tr_at(kK + ro + tx_hi[mb]);
          kt[kk][mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      // Masks first, on S (-inf for keys the rule hides): a branch that rewrites S in place.
      const bool full = j1 < N && wq_last == qw0 + 31 && (p.wr < 0 || j1 <= qw0 + p.wr) &&
                        (p.wl < 0 || j0 >= wq_last - p.wl);
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + key_of_reg(r, hh);
          const bool vis = key < N && qi < N && (p.wr < 0 || key <= qi + p.wr) && (p.wl < 0 || key >= qi - p.wl);
          s[r] = vis ? s[r] : -INFINITY;
        }
      }
      float pr[16];
      if (ALIBI && (j1 <= qw0 || j0 >= wq_last)) {
        // Every key of the tile on one side of every query of the wave: |i - j| = +-(j - i)
        // and j - i = (j0 + 8 hh - qi) + key_of_reg(r, 0), a constant per register.
        const float ss = j1 <= qw0 ? slope2 : -slope2;  // bias = ss * (j - i)
        const float b0 = ss * (float)(j0 + 8 * hh - qi);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pr[r] = fast_exp2(fmaf(s[r], p.scale_log2, fmaf(ss, (float)key_of_reg(r, 0), b0)) - lse2);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float y = s[r] * p.scale_log2;
          if (ALIBI) y = fmaf(-slope2, fabsf((float)(qi - (j0 + key_of_reg(r, hh)))), y);
          pr[r] = fast_exp2(y - lse2);
        }
      }
      // dQ^T += K^T dS^T: A = K^T (read above), B = dS^T from registers.
      // Keep words (register r: word keep_word(r), bit keep_bit(r)).
      uint32_t keep[4] = {};
      if constexpr (DROPOUT) {
        keep_words_qlane(p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_keep, bh, qi, t, hh, keep);
#pragma unroll
        for (int n = 0; n < 4; ++n) opaque(keep[n]);  // unpacked where they are used, not ahead of the MFMAs
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float d8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * kk + e;
          // dropout: pr = P r, dp = dP - D / r; dS = P (Z dP r - D) = pr * (Z ? dp : -D / r)
          d8[e] = DROPOUT ? pr[r] * select_bits(keep_mask_of(keep[keep_word(r)], keep_bit(r)), dp[r], ndelta) : pr[r] * dp[r];
        }
        const bf16x8 dsb = pack_bf16x8(d8[0], d8[1], d8[2], d8[3], d8[4], d8[5], d8[6], d8[7]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32(kt[kk][mb], dsb, acc[mb]);
      }
    }
    wait_ring<NST, 2 * PER_WAVE>(n_tiles - u - 2);  // tile u + 1 has landed
  };

  wait_vm_all();
  static_for<0, NST - 1>([&](auto sc) {
    constexpr int k = decltype(sc)::value;
    if (k < n_tiles) issue(tile_at(k), std::integral_constant<int, k>{});
  });
  wait_ring<NST, 2 * PER_WAVE>(n_tiles - 1);  // the first tile to visit has landed
  for (int u = 0; u < n_tiles; u += NST) {
    static_for<0, NST>([&](auto sc) {
      constexpr int k = decltype(sc)::value;
      if (u + k < n_tiles) body(u + k, sc);
    });
  }
  if (!wave_live || qi >= N) return;
  bf16* dq_row = (bf16*)p.dq + base + (int64_t)qi * rs;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (bf16)(acc[mb][4 * a + e] * p.scale);
      *reinterpret_cast<bf16x4*>(dq_row + 32 * mb + 8 * a + 4 * hh) = x;
    }
  }
}

// ---------------------------------------------------------------- launch
#ifndef FA2_BWD_NW
#define FA2_BWD_NW 4
#endif
#ifndef FA2_BWD_NST
#define FA2_BWD_NST 2
#endif
#ifndef FA2_BWD64_NST
#define FA2_BWD64_NST 3
#endif
#ifndef FA2_DQ64_NST
#define FA2_DQ64_NST 3
#endif
#ifndef FA2_DQ_NW
#define FA2_DQ_NW 4
#endif
#ifndef FA2_DQ_NST
#define FA2_DQ_NST 3
#endif

template <typename K>
static hipError_t set_lds(K kern, int bytes) {
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return e == hipSuccess ? check_lds_at_zero((const void*)kern) : e;
}

// Pass 1: D = rowsum(dO * O); with zero_acc also clears the float32 dQ accumulator.
template <int D>
static hipError_t launch_prep_d(const BwdParams& p, bool zero_acc, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.N * p.H;
  constexpr int RPB = 256 / (D / 8);
  const unsigned row_blocks = (unsigned)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(row_blocks), dim3(256), 0, stream, p, zero_acc ? 1 : 0);
  return hipGetLastError();
}

// Pass 2: the key-block pass (dK, dV; with DET = false also the atomic dQ).
template <int D, bool ALIBI, bool DET, bool VARLEN, bool SPARSE, bool DROPOUT = false>
static hipError_t launch_main_d(const BwdParams& p0, hipStream_t stream) {
  // Split dQ pass (DET): 4 waves per 128-key block, two workgroups per CU (2-stage
  // rings at d = 128, so that both fit in LDS). Each workgroup has its own barriers,
  // so the two drift out of step and one's softmax runs beside the other's MFMAs;
  // one 8-wave workgroup with a 4-stage ring measured 3-4 % slower. Atomic dQ:
  // 4 waves, 2 stages (its dS^T buffer and dQ step need the room).
  constexpr int NW = DET ? (D == 128 ? FA2_BWD_NW : 4) : 4;
  constexpr int NST = DET ? (D == 128 ? FA2_BWD_NST : FA2_BWD64_NST) : 2;
  using S = BwdShape<D, NW, NST, DET>;
  auto kmain = bwd_main_kernel<D, ALIBI, DET, NW, NST, VARLEN, SPARSE, DROPOUT>;
  // + the query-tile list (SPARSE) or 32 keep-mask words per wave (DROPOUT)
  constexpr int lds = S::LDS + (SPARSE ? 2 * (kSparseMaxN / S::BQ) : 0) + (DROPOUT ? NW * 128 : 0);
  static_assert(lds <= 160 * 1024, "LDS budget");
  static const hipError_t attr = set_lds(kmain, lds);  // once per kernel; thread-safe initialisation
  if (attr != hipSuccess) return attr;
  BwdParams p = p0;
  p.nblk = VARLEN ? (int)varlen_block_bound(p.N, p.nseq, S::BK) : (p.N + S::BK - 1) / S::BK;
  hipLaunchKernelGGL(kmain, dim3((unsigned)((int64_t)p.nblk * p.B * p.H)), dim3(S::NT), lds, stream, p);
  return hipGetLastError();
}

// Pass 3 of the split backward: dQ by a sweep over key tiles per query block.
template <int D, bool ALIBI, bool VARLEN, bool SPARSE, bool DROPOUT>
static hipError_t launch_dq_d(const BwdParams& p0, hipStream_t stream) {
  constexpr int DNW = (D == 128 && !SPARSE) ? FA2_DQ_NW : 4;  // block-sparse: one mask row per workgroup
  constexpr int DNST = D == 128 ? FA2_DQ_NST : FA2_DQ64_NST;
  auto kdq = bwd_dq_det_kernel<D, ALIBI, DNW, DNST, VARLEN, SPARSE, DROPOUT>;
  constexpr int DQ_LDS = DNST * 2 * 32 * D * 2 + (SPARSE ? 2 * (kSparseMaxN / 32) : 0);  // ring (+ tile list)
  static const hipError_t attr = set_lds(kdq, DQ_LDS);  // once per kernel; thread-safe initialisation
  if (attr != hipSuccess) return attr;
  BwdParams p = p0;
  p.nblk = VARLEN ? (int)varlen_block_bound(p.N, p.nseq, DNW * 32) : (p.N + DNW * 32 - 1) / (DNW * 32);
  hipLaunchKernelGGL(kdq, dim3((unsigned)((int64_t)p.nblk * p.B * p.H)), dim3(DNW * 64), DQ_LDS, stream, p);
  return hipGetLastError();
}

// Pass 3 of the atomic backward: dQ = scale * accumulator, to bf16.
template <int D>
static hipError_t launch_convert_d(const BwdParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.N * p.H;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_dq_convert_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdParams& p, int d, bool zero_acc, hipStream_t stream) {
  return d == 128 ? launch_prep_d<128>(p, zero_acc, stream) : launch_prep_d<64>(p, zero_acc, stream);
}

template <int D, bool VARLEN, bool SPARSE, bool DROPOUT>
static hipError_t launch_dkdv_v(const BwdParams& p, hipStream_t stream) {
  return p.alibi != nullptr ? launch_main_d<D, true, true, VARLEN, SPARSE, DROPOUT>(p, stream)
                            : launch_main_d<D, false, true, VARLEN, SPARSE, DROPOUT>(p, stream);
}

template <int D, bool VARLEN, bool SPARSE, bool DROPOUT>
static hipError_t launch_dq_v(const BwdParams& p, hipStream_t stream) {
  return p.alibi != nullptr ? launch_dq_d<D, true, VARLEN, SPARSE, DROPOUT>(p, stream)
                            : launch_dq_d<D, false, VARLEN, SPARSE, DROPOUT>(p, stream);
}

template <int D>
static hipError_t launch_dkdv_mode(const BwdParams& p, hipStream_t stream) {
  if (p.block_mask != nullptr) return launch_dkdv_v<D, false, true, false>(p, stream);
  if (p.cu_seqlens != nullptr) return launch_dkdv_v<D, true, false, false>(p, stream);
  if (p.dropout) return launch_dkdv_v<D, false, false, true>(p, stream);
  return launch_dkdv_v<D, false, false, false>(p, stream);
}

template <int D>
static hipError_t launch_dq_mode(const BwdParams& p, hipStream_t stream) {
  if (p.block_mask != nullptr) return launch_dq_v<D, false, true, false>(p, stream);
  if (p.cu_seqlens != nullptr) return launch_dq_v<D, true, false, false>(p, stream);
  if (p.dropout) return launch_dq_v<D, false, false, true>(p, stream);
  return launch_dq_v<D, false, false, false>(p, stream);
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch_dkdv_mode<128>(p, stream) : launch_dkdv_mode<64>(p, stream);
}

hipError_t launch_bwd_dq(const BwdParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch_dq_mode<128>(p, stream) : launch_dq_mode<64>(p, stream);
}

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool split_dq, hipStream_t stream) {
  hipError_t e;
  if (split_dq) {
    // The dQ pass forms D and the per-row values itself (they equal the D pass's bit for
    // bit), so it runs first and the key-block pass reads what it wrote.
    BwdParams pq = p;
    pq.fuse_stats = 1;
    if ((e = launch_bwd_dq(pq, d, stream)) != hipSuccess) return e;
    return launch_bwd_dkdv(p, d, stream);
  }
  if (p.cu_seqlens != nullptr || p.block_mask != nullptr || p.dropout) return hipErrorInvalidValue;  // split dQ only
  if ((e = launch_bwd_prep(p, d, true, stream)) != hipSuccess) return e;
  const bool alibi = p.alibi != nullptr;
  if (d == 128) {
    e = alibi ? launch_main_d<128, true, false, false, false>(p, stream)
              : launch_main_d<128, false, false, false, false>(p, stream);
  } else {
    e = alibi ? launch_main_d<64, true, false, false, false>(p, stream)
              : launch_main_d<64, false, false, false, false>(p, stream);
  }
  if (e != hipSuccess) return e;
  return d == 128 ? launch_convert_d<128>(p, stream) : launch_convert_d<64>(p, stream);
}

}  // namespace fa2
