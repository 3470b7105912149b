// Forward attention with float32 storage and float32 probabilities.
//
// The same tiled online softmax as the bf16 kernel ("AI基础 | Flash Attention",
// sections Tiling分块 and 在线softmax): K/V tiles of 32 keys pass through LDS,
// every lane owns one query row and keeps its running max, running sum and
// unnormalised running output in registers, and divides once at the end.
// The dot products run on the fp32 VALU (every lane reads the same K/V row,
// an LDS broadcast), so nothing is rounded below float32. This path serves
// small float32 problems where the bf16 MFMA path's rounding of P is not
// acceptable; it is not the throughput path.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace fa2 {

template <int D, bool ALIBI>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p) {
  constexpr int BC = 32;
  constexpr int BR = 64;
  __shared__ __attribute__((aligned(16))) float ks[BC][D];
  __shared__ __attribute__((aligned(16))) float vs[BC][D];

  const int bh_count = p.B * p.H;
  const int qb = p.n_qblocks - 1 - (int)(blockIdx.x / bh_count);
  const int bh = (int)(blockIdx.x % bh_count);
  const int b = bh / p.H, h = bh % p.H;
  const int N = p.N;
  const int lane = threadIdx.x;
  const int64_t rs = (int64_t)p.H * D;
  const int64_t base = (int64_t)b * N * rs + (int64_t)h * D;
  const float* qg = (const float*)p.q + base;
  const float* kg = (const float*)p.k + base;
  const float* vg = (const float*)p.v + base;
  float* og = (float*)p.o + base;

  const int q0 = qb * BR;
  const int q_last = min(q0 + BR, N) - 1;
  const int qi = q0 + lane;

  float qv[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    f32x4 x = qi < N ? *reinterpret_cast<const f32x4*>(qg + (int64_t)qi * rs + c) : f32x4{};
    qv[c] = x[0]; qv[c + 1] = x[1]; qv[c + 2] = x[2]; qv[c + 3] = x[3];
  }
  const float slope2 = ALIBI ? p.alibi[h] * kLog2e : 0.f;

  int kv_lo = 0, kv_hi = N;
  if (p.wl >= 0) kv_lo = max(0, q0 - p.wl);
  if (p.wr >= 0) kv_hi = min(N, q_last + p.wr + 1);
  const int t_lo = kv_lo / BC, t_hi = (kv_hi + BC - 1) / BC;

  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m2 = kNoMax, l = 0.f;

  for (int t = t_lo; t < t_hi; ++t) {
    const int j0 = t * BC;
    __syncthreads();
    for (int e = lane * 4; e < BC * D; e += 64 * 4) {
      const int r = e / D, c = e % D;
      const int key = j0 + r;
      f32x4 kx = f32x4{}, vx = f32x4{};
      if (key < N) {
        kx = *reinterpret_cast<const f32x4*>(kg + (int64_t)key * rs + c);
        vx = *reinterpret_cast<const f32x4*>(vg + (int64_t)key * rs + c);
      }
      *reinterpret_cast<f32x4*>(&ks[r][c]) = kx;
      *reinterpret_cast<f32x4*>(&vs[r][c]) = vx;
    }
    __syncthreads();

    float sc[BC];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], ks[jj][c], dot);
      const int key = j0 + jj;
      float y = dot * p.scale_log2;
      if (ALIBI) y -= slope2 * fabsf((float)(qi - key));
      const bool vis = key < N && (p.wr < 0 || key <= qi + p.wr) && (p.wl < 0 || key >= qi - p.wl);
      y = vis ? y : -INFINITY;
      sc[jj] = y;
      mx = fmaxf(mx, y);
    }
    const float cand = fmaxf(m2, mx);
    const float alpha = fast_exp2(m2 - cand);
    m2 = cand;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      const float pv = fast_exp2(sc[jj] - m2);
      l += pv;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(pv, vs[jj][c], acc[c]);
    }
  }

  if (qi < N) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* orow = og + (int64_t)qi * rs;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      *reinterpret_cast<f32x4*>(orow + c) = f32x4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
    }
    p.lse[(int64_t)bh * N + qi] = l > 0.f ? (m2 + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool ALIBI>
static hipError_t launch_f32_cfg(const FwdParams& p0, hipStream_t stream) {
  FwdParams p = p0;
  p.n_qblocks = (p.N + 63) / 64;
  const int64_t nblk = (int64_t)p.n_qblocks * p.B * p.H;
  hipLaunchKernelGGL((fwd_f32_kernel<D, ALIBI>), dim3((unsigned)nblk), dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t stream) {
  const bool alibi = p.alibi != nullptr;
  if (d == 128) return alibi ? launch_f32_cfg<128, true>(p, stream) : launch_f32_cfg<128, false>(p, stream);
  return alibi ? launch_f32_cfg<64, true>(p, stream) : launch_f32_cfg<64, false>(p, stream);
}

}  // namespace fa2
