// C ABI of the attention library: argument validation and dispatch.
// Every check runs before the first HIP call, so a rejected request touches
// neither the device nor the runtime.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/fa2.h"
#include "launch.hpp"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shared shape/option checks. Returns FA2_OK and sets *empty when there is no work.
fa2_status_t check_common(int B, int H, int N, int d, float scale, int wl, int wr, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0 || d <= 0) return FA2_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_INVALID_ARG;
  if (wl < -1 || wr < -1) return FA2_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT32_MAX) return FA2_ERR_INVALID_ARG;
  if ((double)B * N * H * d >= 4.6e18) return FA2_ERR_INVALID_ARG;
  // grid: ceil(N / 64) * B * H blocks must fit a 32-bit grid dimension
  if ((int64_t)((N + 63) / 64) * B * H > (int64_t)UINT32_MAX) return FA2_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) *empty = true;
  return FA2_OK;
}

fa2::FwdParams fwd_params(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                          int H, int N, float scale, int causal, int wl, int wr, const float* alibi) {
  fa2::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.alibi = alibi;
  p.B = B; p.H = H; p.N = N;
  p.scale = scale;
  p.scale_log2 = scale * fa2::kLog2e;
  p.causal = causal ? 1 : 0;
  p.wl = wl;
  p.wr = causal ? 0 : wr;
  return p;
}

fa2_status_t fwd_common(bool f32, const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int N, int d, float scale, int causal, int wl, int wr,
                        const float* alibi, void* stream) {
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, scale, wl, wr, &empty);
  if (st != FA2_OK || empty) return st;
  if (!q || !k || !v || !out || !lse) return FA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return FA2_ERR_INVALID_ARG;
  if (alibi && !aligned4(alibi)) return FA2_ERR_INVALID_ARG;
  fa2::FwdParams p = fwd_params(q, k, v, out, lse, B, H, N, scale, causal, wl, wr, alibi);
  hipError_t e = f32 ? fa2::launch_fwd_f32(p, d, (hipStream_t)stream)
                     : fa2::launch_fwd_bf16(p, d, (hipStream_t)stream);
  return e == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

}  // namespace

extern "C" {

fa2_status_t fa2_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                     int N, int d, float softmax_scale, int causal, int window_left, int window_right,
                     const float* alibi_slopes, void* stream) {
  return fwd_common(false, q, k, v, out, lse, B, H, N, d, softmax_scale, causal, window_left,
                    window_right, alibi_slopes, stream);
}

fa2_status_t fa2_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse, int B,
                         int H, int N, int d, float softmax_scale, int causal, int window_left,
                         int window_right, const float* alibi_slopes, void* stream) {
  return fwd_common(true, q, k, v, out, lse, B, H, N, d, softmax_scale, causal, window_left,
                    window_right, alibi_slopes, stream);
}

size_t fa2_bwd_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  const size_t rows = (size_t)B * H * N;
  return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

fa2_status_t fa2_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                     int causal, int window_left, int window_right, const float* alibi_slopes,
                     int deterministic, void* stream) {
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK || empty) return st;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !workspace)
    return FA2_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, out, lse, dout, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA2_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA2_ERR_INVALID_ARG;
  if (workspace_bytes < fa2_bwd_workspace_size(B, H, N, d)) return FA2_ERR_INVALID_ARG;

  fa2::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.dout = dout;
  p.dq = dq; p.dk = dk; p.dv = dv;
  const size_t rows = (size_t)B * H * N;
  p.dq_acc = reinterpret_cast<float*>(workspace);
  p.delta = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(rows * d * sizeof(float)));
  p.alibi = alibi_slopes;
  p.B = B; p.H = H; p.N = N;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * fa2::kLog2e;
  p.causal = causal ? 1 : 0;
  p.wl = window_left;
  p.wr = causal ? 0 : window_right;
  // The separate dQ pass (no atomics) is both bitwise repeatable and, on MI355X,
  // faster than accumulating dQ with float atomics, so it serves both values of
  // `deterministic`. FA2_BWD_ATOMIC_DQ=1 selects the atomic variant when
  // determinism is not requested (a tuning switch; results stay within tolerance).
  bool split_dq = true;
  if (deterministic == 0) {
    const char* env = getenv("FA2_BWD_ATOMIC_DQ");
    if (env && strcmp(env, "1") == 0) split_dq = false;
  }
  hipError_t e = fa2::launch_bwd_bf16(p, d, split_dq, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return FA2_ERR_UNSUPPORTED;
  return e == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

const char* fa2_status_string(fa2_status_t s) {
  switch (s) {
    case FA2_OK: return "FA2_OK";
    case FA2_ERR_INVALID_ARG: return "FA2_ERR_INVALID_ARG: invalid argument";
    case FA2_ERR_UNSUPPORTED: return "FA2_ERR_UNSUPPORTED: request not supported by this build";
    case FA2_ERR_HIP: return "FA2_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown fa2 status";
}

int fa2_version(void) { return kVersion; }

}  // extern "C"
