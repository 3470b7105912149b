// Forward attention, bf16 storage, on gfx950 MFMA.
//
// Method ("AI基础 | Flash Attention", sections Tiling分块 / 在线softmax /
// Flash Attention2; FlashAttention-2 paper abstract, items (1)-(3)):
// one workgroup per (batch, head, block of BR query rows); the K/V tiles of
// the visible key range stream through LDS; every wavefront owns 32 query rows
// and keeps its running max, running sum and unnormalised running output in
// registers; the output is divided by the running sum once, at the end; only
// O and the per-row logsumexp are written back.
//
// gfx950 mapping (the pages' kernel was written for NVIDIA parts):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with K as the A operand (from
//    LDS) and Q^T as the B operand (registers, loaded once). Each lane then
//    holds the scores of ONE query row (lane % 32) for 16 keys of a 32-key
//    subtile, so the row max / row sum are in-lane plus a single
//    v_permlane32_swap between the two lane halves.
//  * O^T += V^T P^T with P^T as the B operand straight from registers (the K
//    rows are loaded in a permuted order so that each lane half holds eight
//    consecutive keys per 16-key reduction step), and V^T read from the
//    row-major V tile with ds_read_b64_tr_b16. O^T keeps each query's
//    accumulator in the same lanes as its softmax statistics, so the rescale by
//    exp2(m_old - m_new) and the final 1/l are per-lane scalars.
//  * The running max is kept in log2 units (scores times scale*log2 e) and
//    the output is rescaled only when some row's max grew by more than
//    2^kRescaleLog2 — every P then stays <= 2^kRescaleLog2 — which is exact:
//    numerator and denominator share the same reference max.
//  * K/V tiles go straight from global memory into an NST-stage LDS ring
//    (global_load_lds_dwordx4); the loads of tile t + NST - 1 are issued before
//    the MFMAs of tile t, and one barrier per tile hands a stage over. LDS rows
//    are XOR-swizzled in 16-byte chunks so that the 16-byte K reads and the
//    transposed V reads are free of bank conflicts.
//  * Causal / windowed grids run the longest query blocks first, and each XCD
//    walks two neighbouring heads at a time (grid_map), so the workgroups of a
//    head that run together share its K/V tiles in their XCD's L2; masks are
//    evaluated only on tiles that cross a mask edge or the end of the sequence.
//  * VARLEN: sequences of different lengths packed along the token axis (the
//    variable-length batches of the wmrh.cn FlashAttention v2 article, section
//    6). The grid covers an upper bound of the query blocks actually present
//    (not B x the longest sequence); each workgroup finds its sequence from the
//    boundaries (varlen_block) and the few spare workgroups exit at once.
//    Everything after that is the fixed-length code with the sequence's start,
//    length and LSE row.
//  * SPARSE: block-sparse attention (the block-sparse patterns of the same
//    article, section 6) with a byte per 128 x 128 (query block, key block)
//    pair. The workgroup's query block is one mask row; the K/V tiles of its
//    active key blocks are compacted into a list in LDS (compact_tiles) and
//    the ring streams only those, so skipped blocks cost neither loads nor
//    MFMAs. Masks inside a tile are the dense ones.
//  * DROPOUT: dropout on the attention weights (the dropout_p argument of the
//    same article, section 5.1). Each lane runs one Philox4x32-10 call per
//    32-key subtile, for its query and its own sixteen keys of the subtile
//    (keep_words_qlane), and masks the packed bf16 weight pairs with pair masks
//    built by a byte permute; the row sum and LSE use the undropped
//    weights, the P*V operand the kept ones, and 1 / (1 - p) joins 1 / l in
//    the epilogue.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace fa2 {

constexpr float kRescaleLog2 = 8.0f;
#ifndef FA2_HEAD_GROUP
#define FA2_HEAD_GROUP 2
#endif
// Heads walked together per XCD: pairs of neighbouring heads.
constexpr int kHeadGroup = FA2_HEAD_GROUP;

template <int D, int NW, int BC, int NST>
struct FwdShape {
  static constexpr int NT = NW * 64;        // threads
  static constexpr int BR = NW * 32;        // query rows per workgroup
  static constexpr int TILE = BC * D * 2;   // bytes of one K (or V) tile
  static constexpr int NSUB = BC / 32;      // 32-key subtiles per tile
  static constexpr int KS = D / 16;         // MFMA reduction steps over d
  static constexpr int MB = D / 32;         // 32-row blocks of O^T
  static constexpr int STAGE = 2 * TILE;    // K and V of one tile
  static constexpr int LDS = NST * STAGE;   // NST-stage ring: NST - 1 tiles in flight
  static constexpr int PER_WAVE = TILE / (1024 * NW);  // 1 KB direct-load pieces per wave per tensor
  static constexpr int VM_PER_TILE = 2 * PER_WAVE;     // direct loads per wave per tile (K and V)
  static constexpr int ROWB = 2 * D;        // bytes per LDS row
};

// Occupancy hint: with d = 128 and 32-key tiles the LDS ring takes 32 KB per
// workgroup, so three workgroups (3 waves per SIMD, 96 KB of LDS) share a CU.
// Stating the figure lets the scheduler spend up to 168 registers per lane
// instead of saving them for occupancy that would not help: three waves per SIMD
// already keep the LDS port busy while one of them waits on its MFMAs.
#ifndef FA2_FWD_OCC
#define FA2_FWD_OCC 3
#endif
// The dropout variant's generator needs more registers: 2 waves per SIMD.
template <int D, bool DROPOUT>
constexpr int fwd_occupancy() {
  return D == 128 ? (DROPOUT ? 2 : FA2_FWD_OCC) : 2;
}
template <int D, int NW, int BC, int NST, bool ALIBI, bool VARLEN, bool SPARSE, bool DROPOUT>
__global__ __launch_bounds__(NW * 64, (4 * fwd_occupancy<D, DROPOUT>() / NW))
__attribute__((amdgpu_waves_per_eu(D == 128 ? fwd_occupancy<D, DROPOUT>() : 1, D == 128 ? fwd_occupancy<D, DROPOUT>() : 8)))
void fwd_bf16_kernel(FwdParams p) {
  using S = FwdShape<D, NW, BC, NST>;
  static_assert(!(VARLEN && SPARSE), "packed batches have no block mask");
  static_assert(!DROPOUT || !(VARLEN || SPARSE), "dropout runs on fixed-length dense batches");
  static_assert(!SPARSE || S::BR == kSparseBlock, "a workgroup covers one mask row");
  constexpr int PER_WAVE = S::PER_WAVE;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  int bh, qb;
  grid_map<kHeadGroup, true>((int)blockIdx.x, p.n_qblocks, p.B * p.H, true, bh, qb);  // longest first
  int h, N;
  int64_t tok0, stat0;  // first token of the sequence; index of its row 0 in lse
  if constexpr (VARLEN) {
    int t0, len;
    if (!varlen_block(p.cu_seqlens, p.nseq, p.N, S::BR, qb, qb, t0, len)) return;
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

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int g = lane >> 4, j = lane & 15;
  const int64_t rs = (int64_t)p.H * D;  // elements between consecutive tokens
  const int64_t base = tok0 * rs + (int64_t)h * D;
  const bf16* qg = (const bf16*)p.q + base;
  const bf16* kg = (const bf16*)p.k + base;
  const bf16* vg = (const bf16*)p.v + base;
  bf16* og = (bf16*)p.o + base;

  const int q0 = qb * S::BR;
  const int q_last = min(q0 + S::BR, N) - 1;
  const int qw0 = q0 + 32 * w;        // first query row of this wave
  const int qi = qw0 + l32;           // query row of this lane
  const bool wave_live = qw0 < N;
  const int wq_last = min(qw0 + 31, N - 1);

  // Q^T fragments: lane holds q[qi][16*ks + 8*hh .. +7] for every step ks.
  bf16x8 qf[S::KS];
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) {
    qf[ks] = qi < N ? *reinterpret_cast<const bf16x8*>(qg + (int64_t)qi * rs + 16 * ks + 8 * hh) : bf16x8{};
  }
  const float slope2 = ALIBI ? p.alibi[h] * kLog2e : 0.f;

  // Visible key range of the whole block.
  int kv_lo = 0, kv_hi = N;
  if (p.wl >= 0) kv_lo = max(0, q0 - p.wl);
  if (p.wr >= 0) kv_hi = min(N, q_last + p.wr + 1);
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;

  // The tiles to visit: t_lo .. t_hi - 1, or for SPARSE those of active key blocks.
  uint16_t* tile_list = reinterpret_cast<uint16_t*>(smem + S::LDS);
  int n_tiles = t_hi - t_lo;
  if constexpr (SPARSE) {
    const uint8_t* mrow = p.block_mask + (int64_t)(bh / p.H) * p.mask_sb + (int64_t)h * p.mask_sh +
                          (int64_t)qb * p.nbk;
    static_assert(kSparseBlock % BC == 0, "whole tiles per mask block");
    n_tiles = compact_tiles(tile_list, t_lo, t_hi, kSparseBlock / BC, w,
                            [&](int b) -> uint32_t { return mrow[b] != 0 ? 1u : 0u; });
    __syncthreads();
  }
  // Tiles in ascending order: the workgroups of a head that start together read
  // each K/V tile at about the same time, so it is fetched once into L2 (with
  // the pairs of neighbouring heads per XCD this missed least of the orders and
  // groupings measured). Under ALiBi the sweep runs from the last tile down: the
  // bias grows toward the diagonal, so an ascending sweep would raise the row
  // maximum on nearly every tile (and rescale O each time).
  auto tile_at = [&](int u) __attribute__((always_inline)) -> int {
    const int k = ALIBI ? n_tiles - 1 - u : u;
    if constexpr (SPARSE) {
      return __builtin_amdgcn_readfirstlane((int)(tile_list[k] & kTileIndexMask));
    } else {
      return t_lo + k;
    }
  };

  // Per-lane byte offsets of this lane's direct-load pieces, relative to a tile's first row.
  uint32_t dma_off[PER_WAVE];
#pragma unroll
  for (int n = 0; n < PER_WAVE; ++n) {
    const int byte = (w * PER_WAVE + n) * 1024 + 16 * lane;
    const int r = byte / S::ROWB;
    const int cc = ((byte % S::ROWB) >> 4) ^ tile_swz<D>(r);
    dma_off[n] = (uint32_t)(r * rs * 2 + cc * 16);
  }

  // Per-lane LDS bases; every read below is (base ^ small constant) + immediate.
  //  K (A operand of S^T): row kperm(l32) (+32*sub), chunk 2*ks + hh.
  const int kr = kperm(l32);
  uint32_t kbase = kr * S::ROWB + ((hh ^ tile_swz<D>(kr)) << 4);
  //  V (transposed reads): rows 8*hh + j/4 (+4) (+16*(2*sub + kk)), columns 16*(g&1) + 4*(j&3) (+32*mb).
  const int vr0 = 8 * hh + (j >> 2);
  const int c0 = 2 * (g & 1) + ((j & 3) >> 1);
  uint32_t vbase_lo = vr0 * S::ROWB + ((c0 ^ tile_swz<D>(vr0)) << 4) + (j & 1) * 8;
  uint32_t vbase_hi = (vr0 + 4) * S::ROWB + ((c0 ^ tile_swz<D>(vr0 + 4)) << 4) + (j & 1) * 8;

  f32x16 o[S::MB];
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) o[mb] = f32x16{};
  float m2 = kNoMax;                   // running max, log2 units
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // running sum (this lane half's keys), 4 partial sums

  auto issue = [&](int t, auto stage_c) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_c)::value;
    char* kl = smem + st * S::STAGE;
    const int row0 = t * BC;
    if (row0 + BC <= N) {
      const char* kgb = reinterpret_cast<const char*>(kg + (int64_t)row0 * rs);
      const char* vgb = reinterpret_cast<const char*>(vg + (int64_t)row0 * rs);
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        char* dst = kl + (w * PER_WAVE + n) * 1024;
        dma16(kgb, dma_off[n], dst);
        dma16(vgb, dma_off[n], dst + S::TILE);
      }
    } else {  // last, partial tile: clamp rows to the sequence
      dma_tile<D, BC, NW>(kl, kg, rs, row0, N, w, lane);
      dma_tile<D, BC, NW>(kl + S::TILE, vg, rs, row0, N, w, lane);
    }
  };

  // One tile (the u-th to visit) of the online softmax for this wave; the stage is a
  // compile-time constant. Tile u + NST - 1 is issued into the stage freed by tile u - 1.
  auto body = [&](int u, auto stage_c) __attribute__((always_inline)) {
    constexpr int st = decltype(stage_c)::value;
    if (u + NST - 1 < n_tiles) issue(tile_at(u + NST - 1), std::integral_constant<int, (st + NST - 1) % NST>{});
    const int t = tile_at(u);
    // The read addresses of the d-steps and d-blocks (base ^ constant) stay in
    // registers across the loop; under ALiBi the K addresses are formed per tile,
    // as its bias terms need the registers.
    if (ALIBI) opaque(kbase);
    const int j0 = t * BC;
    const int j1 = j0 + BC - 1;
    const bool skip = !wave_live || (p.wr >= 0 && j0 > wq_last + p.wr) || (p.wl >= 0 && j1 < qw0 - p.wl);
    if (!skip) {
      // Stage st holds K at LDS address st * STAGE and V after it (the dynamic
      // buffer starts at address 0: the launcher checks there is no static LDS).

      // S^T = K Q^T for each 32-key subtile. The K fragments of reduction step
      // ks + 1 are read while the MFMAs of step ks run (two register buffers).
      f32x16 s[S::NSUB];
#pragma unroll
      for (int sub = 0; sub < S::NSUB; ++sub) s[sub] = f32x16{};
      bf16x8 ka[2][S::NSUB];
      auto kload = [&](int ks, bf16x8(&dst)[S::NSUB]) __attribute__((always_inline)) {
#pragma unroll
        for (int sub = 0; sub < S::NSUB; ++sub) {
          dst[sub] = lds_read16_at(st * S::STAGE + sub * 32 * S::ROWB + (kbase ^ (ks << 5)));
        }
      };
      kload(0, ka[0]);
      static_for<0, S::KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 1 < S::KS) kload(ks + 1, ka[(ks + 1) & 1]);
#pragma unroll
        for (int sub = 0; sub < S::NSUB; ++sub) s[sub] = mfma32(ka[ks & 1][sub], qf[ks], s[sub]);
      });
      // Keep that order in the schedule: the reads of steps 0 and 1, then per
      // step its MFMAs followed by the reads of the step after next.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * S::NSUB, 0);  // LDS reads
      static_for<0, S::KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, ks + 1 < S::KS ? S::NSUB : 0, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, S::NSUB, 0);                       // MFMAs
      });

      // Keep words of this lane's scores (register r of subtile sub: word keep_word(r), bit keep_bit(r)).
      uint32_t keep[S::NSUB][4] = {};
      if constexpr (DROPOUT) {
#pragma unroll
        for (int sub = 0; sub < S::NSUB; ++sub)
          keep_words_qlane(p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_keep, bh, qi, j0 / 32 + sub, hh,
                           keep[sub]);
      }

      // Bias (ALiBi, in log2 units) and masks; masks only on tiles crossing an edge.
      if (ALIBI) {
        // bias = -slope * |i - j|. When every key of the tile lies on one side of every
        // query of the wave, |i - j| = +-(j - i) and j - i = (j0 + 32 sub + 8 hh - i) +
        // kofs(r) with kofs(r) = key_of_reg(r, hh) - 8 hh a constant: two FMAs per score.
        const bool below = j1 <= qw0;      // keys <= queries
        const bool above = j0 >= wq_last;  // keys >= queries
        if (below || above) {
          const float ss = below ? slope2 : -slope2;  // bias = ss * (j - i)
#pragma unroll
          for (int sub = 0; sub < S::NSUB; ++sub) {
            const float b0 = ss * (float)(j0 + 32 * sub + 8 * hh - qi);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float kofs = (float)(key_of_reg(r, 0));
              s[sub][r] = fmaf(s[sub][r], p.scale_log2, fmaf(ss, kofs, b0));
            }
          }
        } else {
#pragma unroll
          for (int sub = 0; sub < S::NSUB; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + 32 * sub + key_of_reg(r, hh);
              s[sub][r] = fmaf(s[sub][r], p.scale_log2, -slope2 * fabsf((float)(qi - key)));
            }
        }
      }
      const bool full = j1 < N && (p.wr < 0 || j1 <= qw0 + p.wr) && (p.wl < 0 || j0 >= wq_last - p.wl);
      if (!full) {
#pragma unroll
        for (int sub = 0; sub < S::NSUB; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * sub + key_of_reg(r, hh);
            const bool vis = key < N && (p.wr < 0 || key <= qi + p.wr) && (p.wl < 0 || key >= qi - p.wl);
            s[sub][r] = vis ? s[sub][r] : -INFINITY;
          }
      }

      // Row max; rescale the output only when some row's max grew past the threshold.
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < S::NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
      if (!ALIBI) mx *= p.scale_log2;
      mx = max_with_other_half(mx);
      const float cand = fmaxf(m2, mx);
      if (wave_any(cand - m2 > kRescaleLog2)) {
        const float alpha = fast_exp2(m2 - cand);
        m2 = cand;
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[i] *= alpha;
#pragma unroll
        for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      }

      // P = exp2(y - m2); running sum in four independent partial sums; O^T += V^T P^T.
      uint32_t vx_lo[S::MB], vx_hi[S::MB];
#pragma unroll
      for (int mb = 0; mb < S::MB; ++mb) {
        vx_lo[mb] = vbase_lo ^ (mb << 6);
        vx_hi[mb] = vbase_hi ^ (mb << 6);
      }
      // One step per 16 keys (subtile sub = step / 2, half kk = step % 2); the V^T
      // fragments of step + 1 are read while the MFMAs of step run.
      bf16x8 va[2][S::MB];
      auto vload = [&](int step, bf16x8(&dst)[S::MB]) __attribute__((always_inline)) {
        const int rowoff = step * 16 * S::ROWB;
#pragma unroll
        for (int mb = 0; mb < S::MB; ++mb) {
          const bf16x4 lo = lds_read_tr_at(st * S::STAGE + S::TILE + rowoff + vx_lo[mb]);
          const bf16x4 hi = lds_read_tr_at(st * S::STAGE + S::TILE + rowoff + vx_hi[mb]);
          dst[mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      vload(0, va[0]);
      static_for<0, 2 * S::NSUB>([&](auto sc) {
        constexpr int step = decltype(sc)::value;
        constexpr int sub = step / 2, kk = step % 2;
        if constexpr (step + 1 < 2 * S::NSUB) vload(step + 1, va[(step + 1) & 1]);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = s[sub][8 * kk + e];
          pv[e] = ALIBI ? fast_exp2(x - m2) : fast_exp2(fmaf(x, p.scale_log2, -m2));
        }
        // The P*V operand: the kept weights under dropout. Registers 8 kk + 4 n' + b are
        // byte b of keep word 2 kk + n' (bit 7 set: kept); v_perm's sign-of-byte selectors
        // turn two such bytes into the 0xffff halves that mask one packed bf16 pair.
        bf16x8 pb = pack_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        if constexpr (DROPOUT) {
          u32x4 u = __builtin_bit_cast(u32x4, pb);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t wk = keep[sub][2 * kk + (m >> 1)];
            // selector 8: sign of byte 1 of (wk << 8) = byte 0 of wk; 9: byte 2; 10: byte 1 of wk; 11: byte 3
            u[m] &= __builtin_amdgcn_perm(wk, wk << 8, (m & 1) ? 0x0B0B0909u : 0x0A0A0808u);
          }
          pb = __builtin_bit_cast(bf16x8, u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) lsum[e & 3] += pv[e];
#pragma unroll
        for (int mb = 0; mb < S::MB; ++mb) o[mb] = mfma32(va[step & 1][mb], pb, o[mb]);
      });
    }
    // Tile u + 1 must have landed; the tiles issued after it may still be in flight.
    wait_ring<NST, S::VM_PER_TILE>(n_tiles - u - 2);
  };

  wait_vm_all();
  static_for<0, NST - 1>([&](auto sc) {
    constexpr int k = decltype(sc)::value;
    if (k < n_tiles) issue(tile_at(k), std::integral_constant<int, k>{});
  });
  wait_ring<NST, S::VM_PER_TILE>(n_tiles - 1);  // the first tile to visit has landed
  for (int u = 0; u < n_tiles; u += NST) {
    static_for<0, NST>([&](auto sc) {
      constexpr int k = decltype(sc)::value;
      if (u + k < n_tiles) body(u + k, sc);
    });
  }

  if (!wave_live) return;
  const float lt = sum_with_other_half((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
  const float inv = (lt > 0.f ? 1.0f / lt : 0.f) * (DROPOUT ? p.drop_scale : 1.0f);
  if (qi < N) {
    bf16* orow = og + (int64_t)qi * rs;
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 val;
        val[0] = (bf16)(o[mb][4 * a + 0] * inv);
        val[1] = (bf16)(o[mb][4 * a + 1] * inv);
        val[2] = (bf16)(o[mb][4 * a + 2] * inv);
        val[3] = (bf16)(o[mb][4 * a + 3] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * mb + 8 * a + 4 * hh) = val;
      }
    }
    if (hh == 0) p.lse[stat0 + qi] = lt > 0.f ? (m2 + log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, int NW, int BC, int NST, bool ALIBI, bool VARLEN, bool SPARSE, bool DROPOUT>
static hipError_t launch_fwd_cfg(const FwdParams& p0, hipStream_t stream) {
  using S = FwdShape<D, NW, BC, NST>;
  FwdParams p = p0;
  p.n_qblocks = VARLEN ? (int)varlen_block_bound(p.N, p.nseq, S::BR) : (p.N + S::BR - 1) / S::BR;
  auto kern = fwd_bf16_kernel<D, NW, BC, NST, ALIBI, VARLEN, SPARSE, DROPOUT>;
  // SPARSE: room for the tile list after the ring (one uint16 per key tile)
  constexpr int lds = S::LDS + (SPARSE ? 2 * (kSparseMaxN / BC) : 0);
  // Once per kernel (thread-safe initialisation of a local static).
  static const hipError_t attr = [&] {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return e == hipSuccess ? check_lds_at_zero((const void*)kern) : e;
  }();
  if (attr != hipSuccess) return attr;
  const int64_t nblk = (int64_t)p.n_qblocks * p.B * p.H;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(S::NT), lds, stream, p);
  return hipGetLastError();
}

#ifndef FA2_FWD_NW
#define FA2_FWD_NW 4
#endif
#ifndef FA2_FWD_NST
#define FA2_FWD_NST 2
#endif

#ifndef FA2_FWD64_BC
#define FA2_FWD64_BC 64
#endif
#ifndef FA2_FWD_BC
#define FA2_FWD_BC 32
#endif
template <int D, bool VARLEN, bool SPARSE, bool DROPOUT>
static hipError_t launch_fwd_d(const FwdParams& p, hipStream_t stream) {
  constexpr int NW = SPARSE ? kSparseBlock / 32 : FA2_FWD_NW, NST = FA2_FWD_NST, BC = D == 128 ? FA2_FWD_BC : FA2_FWD64_BC;
  return p.alibi != nullptr ? launch_fwd_cfg<D, NW, BC, NST, true, VARLEN, SPARSE, DROPOUT>(p, stream)
                            : launch_fwd_cfg<D, NW, BC, NST, false, VARLEN, SPARSE, DROPOUT>(p, stream);
}

template <int D>
static hipError_t launch_fwd_mode(const FwdParams& p, hipStream_t stream) {
  if (p.block_mask != nullptr) return launch_fwd_d<D, false, true, false>(p, stream);
  if (p.cu_seqlens != nullptr) return launch_fwd_d<D, true, false, false>(p, stream);
  if (p.dropout) return launch_fwd_d<D, false, false, true>(p, stream);
  return launch_fwd_d<D, false, false, false>(p, stream);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch_fwd_mode<128>(p, stream) : launch_fwd_mode<64>(p, stream);
}

}  // namespace fa2
