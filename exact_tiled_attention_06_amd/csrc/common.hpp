// Device helpers for the gfx950 attention kernels: vector types, MFMA and LDS
// transpose-read wrappers, wavefront reductions and launch parameter blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA2_LDS __attribute__((address_space(3)))
#define FA2_GLOBAL __attribute__((address_space(1)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no score seen yet" in the running max, so that
// exp2(m_old - m_new) never evaluates (-inf) - (-inf).
constexpr float kNoMax = -1.0e30f;

// D = A * B + C on a 32x32x16 bf16 tile. Lane l supplies row (A) / column (B)
// l % 32 and 8 consecutive reduction slots for half l / 32. C/D: lane l, reg r
// holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte LDS read at a byte offset from the start of dynamic/static LDS.
__device__ __forceinline__ bf16x8 lds_read16(const char* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

// The same reads at an absolute LDS byte address. Kernels whose only LDS is the
// dynamic buffer see it at address 0 (their launchers check that the kernel has
// no static LDS), so a constant part of the address folds into the
// instruction's offset field instead of costing an add per read.
__device__ __forceinline__ bf16x8 lds_read16_at(uint32_t addr) {
  return *reinterpret_cast<const bf16x8 FA2_LDS*>((uintptr_t)addr);
}
__device__ __forceinline__ f32x4 lds_read_f32x4_at(uint32_t addr) {
  return *reinterpret_cast<const f32x4 FA2_LDS*>((uintptr_t)addr);
}
__device__ __forceinline__ bf16x4 lds_read_tr_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FA2_LDS*)((uintptr_t)addr));
}

// Host side: the absolute-address reads above assume the dynamic LDS buffer
// starts at address 0, i.e. that the kernel declares no static LDS.
inline hipError_t check_lds_at_zero(const void* kernel) {
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, kernel);
  if (e != hipSuccess) return e;
  return fa.sharedSizeBytes == 0 ? hipSuccess : hipErrorInvalidDeviceFunction;
}

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives four
// 16-bit values; value e comes from the 8 bytes addressed by group lane
// 4*e + i/4, element i%4. If group lane j addresses row (r0 + j/4), columns
// (c0 + 4*(j%4) .. +3) of a row-major matrix, lane i receives column c0 + i,
// rows r0 .. r0+3: a 4x16 block read transposed.
__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 FA2_LDS*)(p));
}

// Row max / row sum across the two lane halves (lane l and l ^ 32) with
// v_permlane32_swap: its two results hold this lane's value and the other
// half's (lanes 0..31: own, partner; lanes 32..63: partner, own).
__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight fp32 values -> eight bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// The key (within a 32-key subtile) that C register r of a lane in half hh
// holds after S^T = K Q^T, when A-operand lane m loads key row kperm(m).
// With kperm below, registers 0..7 of half hh are keys 8*hh + 0..7 and
// registers 8..15 are keys 16 + 8*hh + 0..7: eight consecutive keys per
// 16-key reduction step, the layout the P*V step consumes directly.
__device__ __forceinline__ int kperm(int m) {
  const int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}
__host__ __device__ constexpr int key_of_reg(int r, int hh) { return 16 * (r >> 3) + 8 * hh + (r & 7); }

// XOR swizzle of 16-byte chunks in an LDS tile of rows of D bf16 values.
// It keeps two access patterns free of bank conflicts (64 banks x 4 bytes):
//  * 16-byte row reads: 16 lanes read the same chunk of 16 consecutive rows;
//  * transposed reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows
//    (first row a multiple of 4) x 4 consecutive chunks.
// D = 128 (16 chunks per 256-byte row): chunk c of row r sits at c ^ f(r),
// f(r) = 4*(r%4) + (r/4)%4, a bijection on 16 consecutive rows whose high
// part separates the 4 rows of a transposed read.
// D = 64 (8 chunks, two rows per 256 bytes): f(r) = 4*((r/2)%2) + (r/4)%4.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ uint32_t tile_off(int r, int cc) {
  return r * (D * 2) + ((cc ^ tile_swz<D>(r)) << 4);
}
// Byte address of the 8-byte piece (row r, columns col..col+3) for a transposed read.
template <int D>
__device__ __forceinline__ uint32_t tile_off_tr(int r, int col) {
  return tile_off<D>(r, col >> 3) + (col & 7) * 2;
}

// Direct global->LDS loads (gfx950 global_load_lds_dword / _dwordx4): lane i
// of the wave reads its own global address and the data lands in LDS at
// lds_dst + 4*i (dword) or + 16*i (dwordx4); no register receives it. They are
// issued from inline assembly on purpose: the compiler treats its own builtin
// for these loads as an LDS store of unknown extent and fences every later
// transposed LDS read (ds_read_b64_tr_b16) with s_waitcnt vmcnt(0), which
// drains the whole prefetch ring at each tile. Here the kernels track
// completion themselves (wait_vm_and_sync with the ring's exact count; vector
// loads complete in issue order). The asm has no outputs: nothing is written
// to a register while the load is in flight. M0 (the LDS destination) is an
// input the compiler sets; s_nop 0 separates that write from the load.
//   dma16: base (uniform) + voff (per lane, bytes); dma4: a per-lane address.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const char* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const void FA2_LDS*)lds_dst;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* addr, const char* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const void FA2_LDS*)lds_dst;
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "{m0}"(m0) : "memory");
}

// Copies rows [row0, row0 + ROWS) of one head (row stride rs elements) into
// an LDS tile laid out with tile_off, using the direct global->LDS loads
// (PER_WAVE dwordx4 loads per wave). Each lane loads the 16-byte chunk that
// the swizzle places at its LDS slot. Rows at or past n_rows read row
// n_rows - 1 (finite data that the caller masks), so no load leaves the
// tensor; row0 < n_rows. The caller waits (s_waitcnt) and synchronises before
// reading the tile.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(char* lds_tile, const bf16* g, int64_t rs, int row0, int n_rows,
                                         int w, int lane) {
  constexpr int BYTES = ROWS * D * 2;
  constexpr int PER_WAVE = BYTES / (1024 * NW);
  static_assert(BYTES % (1024 * NW) == 0, "tile must split into 1 KB pieces per wave");
  const bf16* tile_base = g + (int64_t)row0 * rs;
#pragma unroll
  for (int n = 0; n < PER_WAVE; ++n) {
    const int m = w * PER_WAVE + n;
    const int byte = m * 1024 + 16 * lane;
    const int r = byte / (2 * D);
    const int slot = (byte % (2 * D)) >> 4;
    const int cc = slot ^ tile_swz<D>(r);
    const int row = min(row0 + r, n_rows - 1);
    dma16(tile_base, (uint32_t)(((row - row0) * rs + cc * 8) * 2), lds_tile + m * 1024);
  }
}

// Wait for every outstanding memory operation of this wave (including direct
// global->LDS loads), then synchronise the workgroup.
__device__ __forceinline__ void wait_all_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Wait for every outstanding vector-memory load of this wave. Called once,
// after the per-lane register loads of a kernel's prologue and before its
// prefetch ring starts: the compiler then knows that no register load is
// pending inside the tile loop and adds no vmcnt wait of its own there (such a
// wait would also drain the ring's direct loads in flight).
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0); expcnt, lgkmcnt: no wait
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (direct global->LDS loads included; they complete in issue order) and all LDS
// operations are done, then synchronise the workgroup.
template <int N>
__device__ __forceinline__ void wait_vm_and_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt[3:0] | expcnt[6:4] (7 = no wait) | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __syncthreads();
}

// Prefetch ring of NST stages, PER direct loads per tile per wave: waits until
// the next tile to compute has landed and synchronises the workgroup.
// `younger` = the number of tiles issued after that one (tile loads complete
// in issue order, so those may stay in flight); it is at most NST - 2 and
// drops to zero or below at the end of the ring, where the wait must cover
// everything.
template <int NST, int PER>
__device__ __forceinline__ void wait_ring(int younger) {
  if constexpr (NST <= 2) {
    wait_vm_and_sync<0>();
  } else {
    if (younger >= NST - 2) {
      wait_vm_and_sync<PER * (NST - 2)>();
    } else {
      wait_ring<NST - 1, PER>(younger);
    }
  }
}

template <int I, int N, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Hides a value from the optimiser so that expressions built from it are
// recomputed where they are used instead of being hoisted (and kept live)
// across a loop.
template <typename T>
__device__ __forceinline__ void opaque(T& x) {
  asm volatile("" : "+v"(x));
}

// Workgroup id -> (head index bh, block index within the head).
//
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), and each XCD
// has its own L2. When bh_count is a multiple of 8 G, XCD x walks its heads G at
// a time: with NEIGHBOURS its g-th group is the G neighbouring heads from
// bh = (8 g + x) G (so the 8 XCDs together hold 8 G neighbouring heads, whose rows
// interleave in memory), else the heads bh = 8 (g G + i) + x, i < G. Within a
// group the blocks run in `order` (longest first), interleaved over the G heads.
// So the workgroups resident on one XCD share few heads and re-read the same K/V
// (or Q/dO) tiles from their L2; which choice misses least depends on the
// kernel's sweep and was measured per kernel. Otherwise the ids map head-fastest.
// `descending`: block index runs nblk-1 .. 0 (causal forward: long blocks are
// the late query blocks); else 0 .. nblk-1 (causal backward: early key blocks).
template <int G, bool NEIGHBOURS = false>
__host__ __device__ __forceinline__ void grid_map(int id, int nblk, int bh_count, bool descending, int& bh, int& blk) {
  int r;
  if ((bh_count & 7) == 0 && ((bh_count >> 3) % G) == 0) {
    const int xcd = id & 7, s = id >> 3;
    const int group = s / (G * nblk), rem = s % (G * nblk);
    r = rem / G;
    bh = NEIGHBOURS ? (group * 8 + xcd) * G + rem % G : ((group * G + rem % G) << 3) + xcd;
  } else {
    r = id / bh_count;
    bh = id % bh_count;
  }
  blk = descending ? nblk - 1 - r : r;
}

// Variable-length batches: nseq sequences packed along the token axis, sequence
// s holding tokens cu[s] .. cu[s+1]-1 of `total`. Blocks of `rows` tokens are
// numbered sequence by sequence (sequence s has ceil(len_s / rows) of them).
// Maps virtual block v to (block index within its sequence, first token,
// length); returns false when v lies past the last block. The 64 lanes of a
// wave take 64 sequences at a time: block counts, an inclusive prefix sum
// across the wave, then a ballot for the first prefix above v. Every wave
// computes the same, uniform answer. Boundaries are clamped into [0, total]
// and each end to at least its start, so malformed offsets cannot address
// memory outside the packed tensors.
__device__ __forceinline__ bool varlen_block(const int* cu, int nseq, int total, int rows, int v, int& blk,
                                             int& tok0, int& len) {
  const int lane = threadIdx.x & 63;
  int rem = v;
  for (int c = 0; c < nseq; c += 64) {
    const int s = c + lane;
    int a = 0, e = 0;
    if (s < nseq) {
      a = min(max(cu[s], 0), total);
      e = min(max(cu[s + 1], a), total);
    }
    const int nb = (e - a + rows - 1) / rows;
    int incl = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > rem);
    if (hit != 0) {
      const int L = __builtin_ctzll(hit);
      blk = __builtin_amdgcn_readfirstlane(rem - (__shfl(incl, L, 64) - __shfl(nb, L, 64)));
      tok0 = __builtin_amdgcn_readfirstlane(__shfl(a, L, 64));
      len = __builtin_amdgcn_readfirstlane(__shfl(e - a, L, 64));
      return true;
    }
    rem -= __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  }
  return false;
}

// Upper bound on the number of virtual blocks of a packed batch: sum over
// sequences of ceil(len_s / rows) <= (total + nseq * (rows - 1)) / rows.
__host__ __device__ inline int64_t varlen_block_bound(int total, int nseq, int rows) {
  return ((int64_t)total + (int64_t)nseq * (rows - 1)) / rows;
}

// Block-sparse attention: one mask byte per (query block, key block) pair of
// kSparseBlock x kSparseBlock positions; zero means the pair is skipped.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxN = 65536;  // bounds the per-workgroup tile list kept in LDS

// Number of lanes below this one whose bit is set in a wave-wide ballot.
__device__ __forceinline__ int lanes_below(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
}

// Compacts the tiles t in [t_lo, t_hi) of the active blocks (tpb tiles per
// block; flags(b), two bits, not zero for an active block b) into list[0 .. n)
// as t | flags << 14 (LDS, in increasing t; wave 0 writes) and returns n. One
// mask read per lane covers 64 blocks, so a row of up to 64 blocks costs one
// memory round trip: each lane's block puts its tiles after those of the lanes
// below it (an inclusive prefix sum across the wave). Tile indices must stay
// below 2^14. Every wave computes the same n; the caller synchronises the
// workgroup before reading the list.
template <typename F>
__device__ __forceinline__ int compact_tiles(uint16_t* list, int t_lo, int t_hi, int tpb, int w, F&& flags) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  if (t_hi <= t_lo) return 0;
  const int b_lo = t_lo / tpb, b_hi = (t_hi - 1) / tpb + 1;
  for (int b0 = b_lo; b0 < b_hi; b0 += 64) {
    const int b = b0 + lane;
    uint32_t f = 0;
    int first = 0, c = 0;
    if (b < b_hi) {
      f = flags(b) & 3u;
      first = max(b * tpb, t_lo);
      c = f != 0 ? min(b * tpb + tpb, t_hi) - first : 0;
    }
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (w == 0) {
      for (int k = 0; k < c; ++k) list[n + incl - c + k] = (uint16_t)((first + k) | (f << 14));
    }
    n += __builtin_amdgcn_readlane(incl, 63);
  }
  return n;
}
constexpr uint32_t kTileIndexMask = (1u << 14) - 1;

// ---------------------------------------------------------------- dropout
// Dropout on the attention weights (the dropout_p argument of section 5.1 of
// the wmrh.cn FlashAttention v2 article; the page names no generator, so the
// keep matrix is defined here): weight (i, j) of head bh = b * H + h is kept
// iff an 8-bit value from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011) is below `keep`
// (keep = round(256 (1 - p)), 0 .. 256). Key (seed mod 2^32, seed div 2^32),
// counter (g, i, bh, offset) with offset < 2^32. A call's sixteen values (its
// output bytes, little-endian) belong to the keys of the 32-key block c = j / 32
// with bit 3 of j equal to g % 2, g = 2 c + that bit, in increasing order: key j
// takes byte 8 ((j / 16) % 2) + j % 8 of group 2 (j / 32) + (j / 8) % 2. These
// are exactly the keys of one lane half in the query-per-lane layout. Kept
// weights are scaled by 1 / (1 - p) where they meet V.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;  // key increments between rounds
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// Ten rounds; each multiplies counter words 0 and 2 by the two constants into
// 64-bit products and mixes their halves with words 1 and 3 and the key.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0, p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// The same register of the lane 32 apart (lane l <-> l ^ 32). permlane32_swap
// returns this lane's value and the other half's value in its two results
// (which is which depends on the half); the XOR of both with the own value is
// the other half's value.
__device__ __forceinline__ uint32_t from_other_half(uint32_t x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] ^ r[1] ^ x;
}

// Keep bits of a 32-bit word of generator output: bit 8 b + 7 is set iff byte
// b is below `keep` (0 .. 256), the other bits are zero. The four bytes are
// compared at once: with h = 0x80 in every byte, (x | h) - (keep & 0x7f) per
// byte never borrows into the next byte, and its bit 7 says
// (b & 0x7f) >= (keep & 0x7f); b < keep is then that bit's complement when b and
// keep agree in bit 7, else keep's bit 7. A host build of this function is
// checked against a plain byte compare for every byte value, position and
// threshold.
__host__ __device__ __forceinline__ uint32_t keep_lt_word(uint32_t x, uint32_t keep) {
  constexpr uint32_t h = 0x80808080u;
  if (keep > 255u) return h;  // p = 0: every weight kept
  const uint32_t lo7 = (keep & 0x7Fu) * 0x01010101u;
  const uint32_t top = (keep & 0x80u) ? 0u : h;  // bytes where a differing bit 7 decides "not below"
  const uint32_t d = (x | h) - lo7;
  return ~((x & d) | ((x ^ d) & top)) & h;
}

// Query-per-lane layout (S^T = K Q^T, A-operand row kperm(m)): lane (query i,
// half hh) holds keys key_of_reg(r, hh) of the 32-key subtile s, which are the
// keys of generator group 2 s + hh, register r taking byte r. Returns in w the
// keep words (keep_lt_word) that hold register r's decision in word keep_word(r)
// at bit keep_bit(r).
__device__ __forceinline__ void keep_words_qlane(uint32_t seed_lo, uint32_t seed_hi, uint32_t offset, uint32_t keep,
                                                 int bh, int i, int s, int hh, uint32_t (&w)[4]) {
  uint32_t x[4];
  philox4x32_10((uint32_t)(2 * s + hh), (uint32_t)i, (uint32_t)bh, offset, seed_lo, seed_hi, x);
#pragma unroll
  for (int n = 0; n < 4; ++n) w[n] = keep_lt_word(x[n], keep);
}
__host__ __device__ constexpr int keep_word(int r) { return r >> 2; }
__host__ __device__ constexpr int keep_bit(int r) { return 8 * (r & 3) + 7; }

// Key-per-lane layout (S = Q K^T, A-operand row kperm(m)): lane (key kw0 + l32,
// half hh) holds queries key_of_reg(r, hh) of the 32-query block at i0;
// kw0 % 32 == 0. Each lane runs the generator for query i0 + l32 and group
// 2 (kw0 / 32) + hh; the halves merge their bits into the query's 32-key row
// mask (byte t of group hh' at bit 8 (t % 4) + 4 hh' + t / 4), which goes to
// slot[l32] (this wave's 32 words of LDS); the block's rows are then read back
// from the slot.
__device__ __forceinline__ void keep_rows_klane(uint32_t seed_lo, uint32_t seed_hi, uint32_t offset, uint32_t keep,
                                                int bh, int i0, int kw0, int l32, int hh, uint32_t* slot) {
  uint32_t x[4];
  philox4x32_10((uint32_t)(2 * (kw0 / 32) + hh), (uint32_t)(i0 + l32), (uint32_t)bh, offset, seed_lo, seed_hi, x);
  uint32_t m = 0;
#pragma unroll
  for (int n = 0; n < 4; ++n) m |= keep_lt_word(x[n], keep) >> (7 - n);  // byte b of word n at bit 8 b + n
  const uint32_t other = from_other_half(m);
  slot[l32] = hh ? (other | (m << 4)) : (m | (other << 4));  // both halves store the same word
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// Bit of key kw0 + l32 in a row mask: byte t = 8 ((l32 / 16) % 2) + l32 % 8 of group (l32 / 8) % 2.
__device__ __forceinline__ int keep_row_bit(int l32) {
  const int t = 8 * ((l32 >> 4) & 1) + (l32 & 7);
  return 8 * (t & 3) + 4 * ((l32 >> 3) & 1) + (t >> 2);
}
// Row mask of register r's query: query key_of_reg(r, hh) of the block, from rows = slot + 8 * hh.
__device__ __forceinline__ uint32_t drop_row(const uint32_t* rows, int r) { return rows[16 * (r >> 3) + (r & 7)]; }

// All ones if bit `pos` of `word` is set, else zero (a sign-extended one-bit field).
__device__ __forceinline__ uint32_t keep_mask_of(uint32_t word, int pos) {
  return (uint32_t)__builtin_amdgcn_sbfe((int)word, pos, 1);
}

// a where mask is all ones, b where it is zero (bitwise, on the float encodings).
__device__ __forceinline__ float select_bits(uint32_t mask, float a, float b) {
  return __uint_as_float((__float_as_uint(a) & mask) | (__float_as_uint(b) & ~mask));
}

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* alibi;  // [H] or null
  int B, H, N;       // packed batches: B = 1, N = total tokens
  int n_qblocks;     // query blocks per head (packed batches: the virtual-block bound)
  const int* cu_seqlens;  // [nseq + 1] sequence boundaries of a packed batch, or null
  int nseq;
  const uint8_t* block_mask;  // block-sparse: mask bytes, or null
  int64_t mask_sb, mask_sh;   // block-sparse: element strides between batches / heads
  int nbk;                    // block-sparse: blocks per side, ceil(N / kSparseBlock)
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  int causal;
  int wl;            // window left (-1 = unbounded)
  int wr;            // window right after the causal clamp (-1 = unbounded)
  int dropout;       // 0: no dropout; else keep iff generator value < drop_keep
  uint32_t drop_keep;
  float drop_scale;  // 1 / (1 - p)
  uint32_t drop_seed_lo, drop_seed_hi, drop_offset;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;  // [B, H, N, d] float32 workspace
  float* ndelta;  // [B, H, N] float32 workspace: -D, D = rowsum(dO * O)
  float* s_init;  // [B, H, N] float32 workspace: -LSE / scale, where the key-block pass starts S
  const float* alibi;
  int B, H, N;       // packed batches: B = 1, N = total tokens
  int nblk;          // blocks per head of the kernel being launched (packed: virtual-block bound)
  const int* cu_seqlens;  // [nseq + 1] sequence boundaries of a packed batch, or null
  int nseq;
  const uint8_t* block_mask;  // block-sparse: mask bytes, or null
  int64_t mask_sb, mask_sh;
  int nbk;
  float scale;
  float scale_log2;
  float inv_scale;
  int causal;
  int wl;
  int wr;
  int dropout;  // as in FwdParams
  uint32_t drop_keep;
  float drop_scale;
  uint32_t drop_seed_lo, drop_seed_hi, drop_offset;
  int fuse_stats;  // dQ pass: form D and write ndelta, s_init itself (needs o), instead of reading them
};

}  // namespace fa2
