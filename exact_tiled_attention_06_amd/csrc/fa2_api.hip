// C ABI of the attention library: argument validation and dispatch.
// Every check runs before the first HIP call, so a rejected request touches
// neither the device nor the runtime.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

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
  // Kernels add windows to positions in 32-bit arithmetic; with windows capped
  // at N - 1 (effective_window) those sums stay below 2N <= 2^31.
  if (N > (1 << 30)) return FA2_ERR_UNSUPPORTED;
  if ((int64_t)B * H > INT32_MAX) return FA2_ERR_INVALID_ARG;
  // The tile loads address a tile's rows as 32-bit byte offsets from its first row:
  // up to 256 rows of H * d bf16 values must span less than 4 GiB.
  if ((int64_t)H * d > (int64_t)1 << 22) return FA2_ERR_UNSUPPORTED;
  if ((double)B * N * H * d >= 4.6e18) return FA2_ERR_INVALID_ARG;
  // grid: ceil(N / 64) * B * H blocks (the most any kernel launches) must fit the
  // signed 32-bit workgroup id the kernels map to (head, block)
  if ((int64_t)((N + 63) / 64) * B * H > (int64_t)INT32_MAX) return FA2_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) *empty = true;
  return FA2_OK;
}

// The window the kernels apply for a problem of n tokens (n = total tokens for
// a packed batch, which bounds every sequence): a side that reaches every key
// (>= n - 1) becomes -1, so no kernel adds an arbitrarily large window to a
// position; causal sets the right side to 0. Inputs are already validated.
void effective_window(int n, int causal, int wl, int wr, int* wl_out, int* wr_out) {
  *wl_out = (wl < 0 || wl >= n - 1) ? -1 : wl;
  *wr_out = causal ? 0 : ((wr < 0 || wr >= n - 1) ? -1 : wr);
}

fa2::FwdParams fwd_params(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                          int H, int N, float scale, int causal, int wl, int wr, const float* alibi) {
  fa2::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.alibi = alibi;
  p.B = B; p.H = H; p.N = N;
  p.scale = scale;
  p.scale_log2 = scale * fa2::kLog2e;
  p.causal = causal ? 1 : 0;
  effective_window(N, causal, wl, wr, &p.wl, &p.wr);
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
  return 2 * align256(rows * sizeof(float)) + align256(rows * d * sizeof(float));
}

}  // extern "C"

namespace {

// Workspace: -D per row, -LSE / scale per row, then (atomic dQ only) the dQ accumulator.
void set_workspace(fa2::BwdParams* p, const void* workspace, size_t rows) {
  char* ws = reinterpret_cast<char*>(const_cast<void*>(workspace));
  p->ndelta = reinterpret_cast<float*>(ws);
  p->s_init = reinterpret_cast<float*>(ws + align256(rows * sizeof(float)));
  p->dq_acc = reinterpret_cast<float*>(ws + 2 * align256(rows * sizeof(float)));
}

// Shared validation of the backward entry points; fills the parameter block.
// need_* say which pointers the entry point reads or writes.
fa2_status_t bwd_setup(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, const void* workspace,
                       size_t workspace_bytes, size_t workspace_need, int B, int H, int N, int d,
                       float scale, int causal, int wl, int wr, const float* alibi, bool need_qkv,
                       bool need_out, bool need_dq, bool need_dkdv, fa2::BwdParams* p, bool* empty) {
  fa2_status_t st = check_common(B, H, N, d, scale, wl, wr, empty);
  if (st != FA2_OK || *empty) return st;
  const void* needed[] = {need_qkv ? q : dout, need_qkv ? k : dout, need_qkv ? v : dout,
                          (const void*)lse, need_out ? out : dout, dout,
                          need_dq ? dq : dout, need_dkdv ? dk : dout, need_dkdv ? dv : dout, workspace};
  for (const void* ptr : needed)
    if (!ptr || !aligned16(ptr)) return FA2_ERR_INVALID_ARG;
  if (alibi && !aligned4(alibi)) return FA2_ERR_INVALID_ARG;
  if (workspace_bytes < workspace_need) return FA2_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * N;
  *p = fa2::BwdParams{};
  p->q = q; p->k = k; p->v = v; p->o = out; p->lse = lse; p->dout = dout;
  p->dq = dq; p->dk = dk; p->dv = dv;
  set_workspace(p, workspace, rows);
  p->alibi = alibi;
  p->B = B; p->H = H; p->N = N;
  p->scale = scale;
  p->scale_log2 = scale * fa2::kLog2e;
  p->inv_scale = 1.0f / scale;
  p->causal = causal ? 1 : 0;
  effective_window(N, causal, wl, wr, &p->wl, &p->wr);
  return FA2_OK;
}

// Workspace of the split backward: -D and -LSE / scale, one float each per row.
size_t stat_bytes(int B, int H, int N) { return 2 * align256((size_t)B * H * N * sizeof(float)); }

fa2_status_t hip_status(hipError_t e) { return e == hipSuccess ? FA2_OK : FA2_ERR_HIP; }

}  // namespace

extern "C" {

fa2_status_t fa2_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                     int causal, int window_left, int window_right, const float* alibi_slopes,
                     int deterministic, void* stream) {
  // The separate dQ pass (no atomics) is both bitwise repeatable and, on MI355X,
  // faster than accumulating dQ with float atomics, so it serves both values of
  // `deterministic`. FA2_BWD_ATOMIC_DQ=1 selects the atomic variant when
  // determinism is not requested (a tuning switch; results stay within tolerance).
  bool split_dq = true;
  if (deterministic == 0) {
    const char* env = getenv("FA2_BWD_ATOMIC_DQ");
    if (env && strcmp(env, "1") == 0) split_dq = false;
  }
  fa2::BwdParams p;
  bool empty = false;
  const size_t need = split_dq ? stat_bytes(B, H, N) : fa2_bwd_workspace_size(B, H, N, d);
  fa2_status_t st = bwd_setup(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, need, B, H, N, d,
                              softmax_scale, causal, window_left, window_right, alibi_slopes, true, true, true,
                              true, &p, &empty);
  if (st != FA2_OK || empty) return st;
  return hip_status(fa2::launch_bwd_bf16(p, d, split_dq, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_prep(const void* out, const void* dout, const float* lse, void* workspace,
                          size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale, void* stream) {
  fa2::BwdParams p;
  bool empty = false;
  fa2_status_t st = bwd_setup(nullptr, nullptr, nullptr, out, lse, dout, nullptr, nullptr, nullptr, workspace,
                              workspace_bytes, stat_bytes(B, H, N), B, H, N, d, softmax_scale, 0, -1, -1, nullptr,
                              false, true, false, false, &p, &empty);
  if (st != FA2_OK || empty) return st;
  return hip_status(fa2::launch_bwd_prep(p, d, false, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dk,
                          void* dv, const void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                          float softmax_scale, int causal, int window_left, int window_right,
                          const float* alibi_slopes, void* stream) {
  fa2::BwdParams p;
  bool empty = false;
  fa2_status_t st = bwd_setup(q, k, v, nullptr, lse, dout, nullptr, dk, dv, workspace, workspace_bytes,
                              stat_bytes(B, H, N), B, H, N, d, softmax_scale, causal, window_left, window_right,
                              alibi_slopes, true, false, false, true, &p, &empty);
  if (st != FA2_OK || empty) return st;
  return hip_status(fa2::launch_bwd_dkdv(p, d, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout, void* dq,
                        const void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                        float softmax_scale, int causal, int window_left, int window_right,
                        const float* alibi_slopes, void* stream) {
  fa2::BwdParams p;
  bool empty = false;
  fa2_status_t st = bwd_setup(q, k, v, nullptr, lse, dout, dq, nullptr, nullptr, workspace, workspace_bytes,
                              stat_bytes(B, H, N), B, H, N, d, softmax_scale, causal, window_left, window_right,
                              alibi_slopes, true, false, true, false, &p, &empty);
  if (st != FA2_OK || empty) return st;
  return hip_status(fa2::launch_bwd_dq(p, d, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_dq_stats(const void* q, const void* k, const void* v, const void* out, const float* lse,
                              const void* dout, void* dq, void* workspace, size_t workspace_bytes, int B, int H,
                              int N, int d, float softmax_scale, int causal, int window_left, int window_right,
                              const float* alibi_slopes, void* stream) {
  fa2::BwdParams p;
  bool empty = false;
  fa2_status_t st = bwd_setup(q, k, v, out, lse, dout, dq, nullptr, nullptr, workspace, workspace_bytes,
                              stat_bytes(B, H, N), B, H, N, d, softmax_scale, causal, window_left, window_right,
                              alibi_slopes, true, true, true, false, &p, &empty);
  if (st != FA2_OK || empty) return st;
  p.fuse_stats = 1;
  return hip_status(fa2::launch_bwd_dq(p, d, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Checks shared by the packed (variable-length) entry points. The packed
// tensors are handed to the fixed-length checks as one batch of `total` tokens.
fa2_status_t check_varlen(const int* cu_seqlens, int B, int total, int H, int d, float scale, int wl, int wr,
                          bool* empty) {
  *empty = false;
  if (B < 0 || total < 0 || B == INT32_MAX) return FA2_ERR_INVALID_ARG;
  if (B == 0 && total > 0) return FA2_ERR_INVALID_ARG;  // no sequence can hold the tokens
  fa2_status_t st = check_common(1, H, total, d, scale, wl, wr, empty);
  if (st != FA2_OK) return st;
  // virtual-block bound (largest for 32-row blocks) times H must fit the grid
  if (fa2::varlen_block_bound(total, B, 32) * H > (int64_t)INT32_MAX) return FA2_ERR_UNSUPPORTED;
  if (B == 0) *empty = true;
  if (*empty) return FA2_OK;
  if (!cu_seqlens || !aligned4(cu_seqlens)) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

}  // namespace

extern "C" {

fa2_status_t fa2_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int* cu_seqlens, int B, int total_tokens, int H, int d, float softmax_scale,
                            int causal, int window_left, int window_right, const float* alibi_slopes,
                            void* stream) {
  bool empty = false;
  fa2_status_t st = check_varlen(cu_seqlens, B, total_tokens, H, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK || empty) return st;
  if (!q || !k || !v || !out || !lse) return FA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return FA2_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA2_ERR_INVALID_ARG;
  fa2::FwdParams p = fwd_params(q, k, v, out, lse, 1, H, total_tokens, softmax_scale, causal, window_left,
                                window_right, alibi_slopes);
  p.cu_seqlens = cu_seqlens;
  p.nseq = B;
  return hip_status(fa2::launch_fwd_bf16(p, d, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens, void* workspace,
                            size_t workspace_bytes, int B, int total_tokens, int H, int d, float softmax_scale,
                            int causal, int window_left, int window_right, const float* alibi_slopes,
                            void* stream) {
  bool empty = false;
  fa2_status_t st = check_varlen(cu_seqlens, B, total_tokens, H, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK || empty) return st;
  fa2::BwdParams p;
  st = bwd_setup(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, stat_bytes(1, H, total_tokens), 1,
                 H, total_tokens, d, softmax_scale, causal, window_left, window_right, alibi_slopes, true, true, true,
                 true, &p, &empty);
  if (st != FA2_OK || empty) return st;
  p.cu_seqlens = cu_seqlens;
  p.nseq = B;
  return hip_status(fa2::launch_bwd_bf16(p, d, true, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Checks shared by the block-sparse entry points (after the dense checks).
fa2_status_t check_block_mask(const unsigned char* block_mask, int N, long long stride_b, long long stride_h) {
  if (N > fa2::kSparseMaxN) return FA2_ERR_UNSUPPORTED;
  if (!block_mask || stride_b < 0 || stride_h < 0) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

template <typename P>
void set_block_mask(P* p, const unsigned char* block_mask, int N, long long stride_b, long long stride_h) {
  p->block_mask = block_mask;
  p->mask_sb = stride_b;
  p->mask_sh = stride_h;
  p->nbk = (N + fa2::kSparseBlock - 1) / fa2::kSparseBlock;
}

}  // namespace

extern "C" {

fa2_status_t fa2_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                                 int N, int d, float softmax_scale, int causal, int window_left, int window_right,
                                 const float* alibi_slopes, const unsigned char* block_mask,
                                 long long mask_stride_b, long long mask_stride_h, void* stream) {
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK || empty) return st;
  if ((st = check_block_mask(block_mask, N, mask_stride_b, mask_stride_h)) != FA2_OK) return st;
  if (!q || !k || !v || !out || !lse) return FA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return FA2_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA2_ERR_INVALID_ARG;
  fa2::FwdParams p = fwd_params(q, k, v, out, lse, B, H, N, softmax_scale, causal, window_left, window_right,
                                alibi_slopes);
  set_block_mask(&p, block_mask, N, mask_stride_b, mask_stride_h);
  return hip_status(fa2::launch_fwd_bf16(p, d, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_blocksparse(const void* q, const void* k, const void* v, const void* out, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                 size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                                 int causal, int window_left, int window_right, const float* alibi_slopes,
                                 const unsigned char* block_mask, long long mask_stride_b,
                                 long long mask_stride_h, void* stream) {
  fa2::BwdParams p;
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK || empty) return st;
  if ((st = check_block_mask(block_mask, N, mask_stride_b, mask_stride_h)) != FA2_OK) return st;
  st = bwd_setup(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, stat_bytes(B, H, N), B, H, N, d,
                 softmax_scale, causal, window_left, window_right, alibi_slopes, true, true, true, true, &p, &empty);
  if (st != FA2_OK || empty) return st;
  set_block_mask(&p, block_mask, N, mask_stride_b, mask_stride_h);
  return hip_status(fa2::launch_bwd_bf16(p, d, true, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// dropout_p in [0, 1): keep threshold floor((1 - p) * 256 + 0.5) on the
// generator's 8-bit values, scale 1 / (1 - p). p = 0 keeps every weight and is
// the dense computation, so it takes the dense kernels.
// offset is the generator's fourth 32-bit counter word, so it must be below 2^32.
fa2_status_t check_dropout(float dropout_p, unsigned long long offset) {
  if (!(dropout_p >= 0.f) || !(dropout_p < 1.f)) return FA2_ERR_INVALID_ARG;
  if (offset > 0xFFFFFFFFull) return FA2_ERR_INVALID_ARG;
  return FA2_OK;
}

template <typename P>
void set_dropout(P* p, float dropout_p, unsigned long long seed, unsigned long long offset) {
  if (dropout_p == 0.f) return;
  p->dropout = 1;
  p->drop_keep = (uint32_t)floor((1.0 - (double)dropout_p) * 256.0 + 0.5);
  p->drop_scale = 1.0f / (1.0f - dropout_p);
  p->drop_seed_lo = (uint32_t)seed;
  p->drop_seed_hi = (uint32_t)(seed >> 32);
  p->drop_offset = (uint32_t)offset;
}

}  // namespace

extern "C" {

fa2_status_t fa2_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                             int N, int d, float softmax_scale, int causal, int window_left, int window_right,
                             const float* alibi_slopes, float dropout_p, unsigned long long seed,
                             unsigned long long offset, void* stream) {
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK) return st;
  if ((st = check_dropout(dropout_p, offset)) != FA2_OK || empty) return st;
  if (!q || !k || !v || !out || !lse) return FA2_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return FA2_ERR_INVALID_ARG;
  if (alibi_slopes && !aligned4(alibi_slopes)) return FA2_ERR_INVALID_ARG;
  fa2::FwdParams p = fwd_params(q, k, v, out, lse, B, H, N, softmax_scale, causal, window_left, window_right,
                                alibi_slopes);
  set_dropout(&p, dropout_p, seed, offset);
  return hip_status(fa2::launch_fwd_bf16(p, d, (hipStream_t)stream));
}

fa2_status_t fa2_bwd_dropout(const void* q, const void* k, const void* v, const void* out, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             int B, int H, int N, int d, float softmax_scale, int causal, int window_left,
                             int window_right, const float* alibi_slopes, float dropout_p,
                             unsigned long long seed, unsigned long long offset, void* stream) {
  fa2::BwdParams p;
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK) return st;
  if ((st = check_dropout(dropout_p, offset)) != FA2_OK || empty) return st;
  st = bwd_setup(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, stat_bytes(B, H, N), B, H, N, d,
                 softmax_scale, causal, window_left, window_right, alibi_slopes, true, true, true, true, &p, &empty);
  if (st != FA2_OK || empty) return st;
  set_dropout(&p, dropout_p, seed, offset);
  return hip_status(fa2::launch_bwd_bf16(p, d, true, (hipStream_t)stream));
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

// ---------------------------------------------------------------------------
// The allocation-free backward. Its per-row workspace (-D and -LSE / scale, the
// only scratch the atomic-free backward uses) lives in a file-scope device array
// that every GPU the library runs on holds until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a stand-in):
// the device address comes from hipGetSymbolAddress, once per device, with that
// device current, and is kept per device.
namespace {

constexpr size_t kScratchRows = size_t(1) << 21;                  // B * H * N at most
constexpr size_t kScratchBytes = 2 * kScratchRows * sizeof(float);  // 16 MiB
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

hipError_t scratch_address(void** out) {
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] { err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)); });
  if (err[dev] != hipSuccess) return err[dev];
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

fa2_status_t fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                             float softmax_scale, int causal, int window_left, int window_right,
                             const float* alibi_slopes, void* stream) {
  bool empty = false;
  fa2_status_t st = check_common(B, H, N, d, softmax_scale, window_left, window_right, &empty);
  if (st != FA2_OK || empty) return st;
  const size_t rows = (size_t)B * H * N;
  if (rows > kScratchRows) return FA2_ERR_UNSUPPORTED;
  // Validate every argument before the first HIP call; the stand-in workspace
  // address is replaced by the device's scratch address below.
  fa2::BwdParams p;
  static const char kStandIn alignas(256) = 0;
  st = bwd_setup(q, k, v, out, lse, dout, dq, dk, dv, &kStandIn, kScratchBytes, stat_bytes(B, H, N), B, H, N, d,
                 softmax_scale, causal, window_left, window_right, alibi_slopes, true, true, true, true, &p, &empty);
  if (st != FA2_OK || empty) return st;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return FA2_ERR_HIP;
  set_workspace(&p, ws, rows);
  return hip_status(fa2::launch_bwd_bf16(p, d, true, (hipStream_t)stream));
}

fa2_status_t fa2_effective_window(int n, int causal, int window_left, int window_right, int* left_out,
                                  int* right_out) {
  if (n < 0 || window_left < -1 || window_right < -1 || !left_out || !right_out) return FA2_ERR_INVALID_ARG;
  effective_window(n, causal, window_left, window_right, left_out, right_out);
  return FA2_OK;
}

}  // extern "C"
