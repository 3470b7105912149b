/*
 * fa2.h -- C ABI of an MI355X (gfx950) exact-attention library in the
 * FlashAttention-2 style: tiled, online softmax, the N x N score matrix never
 * reaches HBM, the forward keeps one logsumexp per row and the backward
 * recomputes the scores from it.
 *
 * What is computed (for every batch b, head h, query row i):
 *   S_ij  = softmax_scale * <q_i, k_j> - slope_h * |i - j|      (key j visible)
 *   S_ij  = -inf                                                 (key j masked)
 *   LSE_i = ln sum_j exp(S_ij)
 *   O_i   = sum_j exp(S_ij - LSE_i) v_j
 * Sources: "AI基础 | Flash Attention" (sections on standard attention, tiling,
 * online softmax and backward recomputation); the FlashAttention-2 paper
 * abstract ("Faster Attention with Better Parallelism and Work Partitioning"):
 * the result is exact, no approximation; the wmrh.cn FlashAttention v2 article,
 * section 5.1 (API changes): softmax_scale, causal, window_size (-1 = unbounded)
 * and alibi_slopes.
 *
 * Visibility of key j to query i (bounds inclusive):
 *   (!causal || j <= i) && (window_left < 0 || j >= i - window_left)
 *                       && (window_right' < 0 || j <= i + window_right'),
 * where window_right' = 0 when causal, else window_right.
 *
 * Conventions shared by every entry point
 *   - Layouts: q, k, v, out, dout, dq, dk, dv are contiguous [B, N, H, d]
 *     (token-major, heads interleaved); lse is contiguous [B, H, N] float32
 *     (natural log); alibi_slopes is [H] float32 or NULL (no bias).
 *   - Memory: every pointer is DEVICE memory allocated and owned by the
 *     caller. The library allocates nothing, frees nothing, keeps no state
 *     between calls and is safe to call from several host threads.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream). All work is queued on it and the call returns at once; a
 *     kernel fault surfaces at the caller's next synchronisation.
 *   - Errors: arguments are validated before any HIP call; on error nothing
 *     is launched and the status says why. B, H or N equal to 0 is an empty
 *     problem: FA2_OK, nothing launched, pointers not inspected.
 *   - Alignment: every tensor pointer must be 16-byte aligned.
 *   - Supported shapes: d in {64, 128}; any N >= 1 (ragged tails masked);
 *     B * H <= 2^31 - 1; B * N * H * d < 2^62; H * d <= 2^22, N <= 2^30 and
 *     ceil(N / 64) * B * H <= 2^31 - 1 (else FA2_ERR_UNSUPPORTED: tiles are
 *     addressed with 32-bit row offsets, positions plus windows with 32-bit
 *     integers, and workgroups by a signed 32-bit id).
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA2_OK = 0,
  FA2_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad window, bad scale, misalignment */
  FA2_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement (e.g. d not in {64,128}) */
  FA2_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} fa2_status_t;

/*
 * Forward, bf16 storage, fp32 accumulation.
 * q, k, v: bf16 [B, N, H, d] (read); out: bf16 [B, N, H, d] (written, O rounded
 * to nearest even); lse: float32 [B, H, N] (written).
 * softmax_scale must be finite and > 0 (the Python wrapper maps None to
 * 1/sqrt(d)). window_left / window_right >= -1. causal != 0 means j <= i.
 * Source: the online-softmax forward of "AI基础 | Flash Attention" (sections
 * Tiling分块, 在线softmax, Flash Attention2) with the section 5.1 parameters of
 * the wmrh.cn FlashAttention v2 article.
 */
fa2_status_t fa2_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int H, int N, int d, float softmax_scale, int causal,
                     int window_left, int window_right, const float* alibi_slopes,
                     void* stream);

/* Forward with float32 storage (q, k, v, out all float32); same arguments and
 * semantics as fa2_fwd. P is kept in float32 (no bf16 rounding anywhere). */
fa2_status_t fa2_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                         int B, int H, int N, int d, float softmax_scale, int causal,
                         int window_left, int window_right, const float* alibi_slopes,
                         void* stream);

/*
 * Bytes of device workspace for the backward at this shape: two per-row float32
 * arrays [B, H, N], -D (D = rowsum(dO * O)) at offset 0 and -LSE / scale after
 * it, then a float32 dQ accumulator [B, H, N, d] used only by the atomic
 * variant (each part rounded up to 256 bytes). The default fa2_bwd and the
 * pass entry points below only touch the two per-row arrays,
 * 2 * round_up(4 * B * H * N, 256) bytes, and accept a workspace of that size.
 * Returns 0 for an empty or invalid shape.
 */
size_t fa2_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward, bf16 storage. Gradients of sum(out * dout) with respect to q, k, v,
 * recomputing the scores from q, k, v and the forward's lse (the recompute
 * idea of "AI基础 | Flash Attention", section 反向传播):
 *   P = exp(S - LSE), dV = P^T dO, dP = dO V^T, D = rowsum(dO * O),
 *   dS = P * (dP - D), dQ = scale * dS K, dK = scale * dS^T Q.
 * q, k, v, out, dout: bf16 [B, N, H, d] (read); lse: float32 [B, H, N] (read,
 * as written by fa2_fwd with the same arguments); dq, dk, dv: bf16 [B, N, H, d]
 * (written). workspace: device memory (see fa2_bwd_workspace_size;
 * workspace_bytes says how much was given; too little is FA2_ERR_INVALID_ARG);
 * its contents need not be initialised and are overwritten.
 * deterministic != 0 guarantees bitwise-repeatable results: dQ is
 * formed by a separate pass over query blocks, without atomics (it runs
 * first and also forms D; then the dK/dV pass). With
 * deterministic = 0 the library may choose; it currently uses the same pass
 * (the faster one on MI355X). Setting the environment variable
 * FA2_BWD_ATOMIC_DQ=1 makes deterministic = 0 accumulate dQ with float32
 * atomics instead, in which case dq may differ in the last bits between runs.
 * No gradient is produced for the ALiBi slopes.
 */
fa2_status_t fa2_bwd(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int H, int N, int d, float softmax_scale, int causal,
                     int window_left, int window_right, const float* alibi_slopes,
                     int deterministic, void* stream);

/*
 * The three passes of the atomic-free backward as separate calls, for callers
 * that schedule them themselves (for instance the dK/dV and dQ passes on two
 * streams: both depend only on fa2_bwd_prep). fa2_bwd itself runs the two-call
 * form fa2_bwd_dq_stats then fa2_bwd_dkdv (below), which saves the extra read
 * of dO. Arguments
 * mean what they mean for fa2_bwd; the same workspace (at least
 * 2 * round_up(4 * B * H * N, 256) bytes) must be passed to all three, with the
 * same lse and softmax_scale, and fa2_bwd_prep must have completed before the
 * other two read it.
 *   fa2_bwd_prep: -D (D = rowsum(dO * O)) and -LSE / scale per row into the
 *                 workspace.
 *   fa2_bwd_dkdv: dK and dV, one pass over query blocks per key block
 *                 (recomputes P and dS; reads both workspace arrays, which
 *                 stand in for lse there; lse is still checked).
 *   fa2_bwd_dq:   dQ, one pass over key tiles per query block (recomputes P and
 *                 dS; reads lse and -D); no atomics, bitwise repeatable.
 * Source: the backward-by-recomputation of "AI基础 | Flash Attention"
 * (section 反向传播), split by output.
 */
fa2_status_t fa2_bwd_prep(const void* out, const void* dout, const float* lse, void* workspace,
                          size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                          void* stream);
fa2_status_t fa2_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dk, void* dv, const void* workspace,
                          size_t workspace_bytes, int B, int H, int N, int d, float softmax_scale,
                          int causal, int window_left, int window_right,
                          const float* alibi_slopes, void* stream);
fa2_status_t fa2_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq, const void* workspace, size_t workspace_bytes,
                        int B, int H, int N, int d, float softmax_scale, int causal,
                        int window_left, int window_right, const float* alibi_slopes,
                        void* stream);

/*
 * The dQ pass with fa2_bwd_prep folded in, as fa2_bwd runs it: besides dQ it
 * forms D = rowsum(dO * O) for every query row it covers and writes -D and
 * -LSE / scale into the workspace, bit for bit what fa2_bwd_prep writes, so
 * that fa2_bwd_dkdv can follow it (on the same stream, or after it completes).
 * fa2_bwd's default algorithm is exactly fa2_bwd_dq_stats then fa2_bwd_dkdv.
 * Arguments as for fa2_bwd_dq, plus out (the forward's output, [B, N, H, d]
 * bf16); the workspace is written. Errors as for fa2_bwd_dq (out null or
 * misaligned: FA2_ERR_INVALID_ARG).
 * Source: the backward-by-recomputation of "AI基础 | Flash Attention"
 * (section 反向传播); D is the rowsum term of its dS formula.
 */
fa2_status_t fa2_bwd_dq_stats(const void* q, const void* k, const void* v, const void* out, const float* lse,
                              const void* dout, void* dq, void* workspace, size_t workspace_bytes, int B,
                              int H, int N, int d, float softmax_scale, int causal, int window_left,
                              int window_right, const float* alibi_slopes, void* stream);

/*
 * Variable-length batches: B sequences of different lengths packed along the
 * token axis, with no padding. The wmrh.cn FlashAttention v2 article (section
 * 6, future directions) names variable-length sequences, handled with
 * padding-aware scheduling, as the method's open inefficiency; the page gives
 * no interface, so this one is:
 *   - q, k, v, out, dout, dq, dk, dv: contiguous [total_tokens, H, d] bf16;
 *   - cu_seqlens: DEVICE int32 [B + 1], cu_seqlens[0] = 0, non-decreasing,
 *     cu_seqlens[B] = total_tokens; sequence b holds tokens cu_seqlens[b] ..
 *     cu_seqlens[b + 1] - 1 and may be empty. The library cannot check the
 *     contents without a synchronisation: other contents give unspecified
 *     results, but every access stays inside the packed tensors (offsets are
 *     clamped into [0, total_tokens]);
 *   - lse (and the backward's D in the workspace): float32 [H, total_tokens];
 *   - every sequence is its own attention problem: a query sees only the keys
 *     of its own sequence, and positions for causal, window_left/right and
 *     ALiBi count from the sequence's first token. Queries and keys share the
 *     boundaries (self-attention).
 * Only the query blocks present are scheduled: the grid covers
 * (total_tokens + B * (rows - 1)) / rows blocks per head for a kernel of
 * `rows`-token blocks, and each workgroup finds its sequence on the device.
 * B = 0 with total_tokens = 0, total_tokens = 0 or H = 0 is an empty problem
 * (FA2_OK, nothing launched); B = 0 with total_tokens > 0 is
 * FA2_ERR_INVALID_ARG. Other arguments and errors as for fa2_fwd / fa2_bwd.
 */
fa2_status_t fa2_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int* cu_seqlens, int B, int total_tokens, int H, int d,
                            float softmax_scale, int causal, int window_left, int window_right,
                            const float* alibi_slopes, void* stream);

/*
 * Backward of fa2_fwd_varlen (same arguments, plus dout, dq, dk, dv and a
 * workspace of at least 2 * round_up(4 * H * total_tokens, 256) bytes, which
 * fa2_bwd_workspace_size(1, H, total_tokens, d) covers). Always the
 * atomic-free algorithm (the dQ pass, which also forms D, then the dK/dV
 * pass): bitwise repeatable.
 */
fa2_status_t fa2_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            const int* cu_seqlens, void* workspace, size_t workspace_bytes,
                            int B, int total_tokens, int H, int d, float softmax_scale, int causal,
                            int window_left, int window_right, const float* alibi_slopes,
                            void* stream);

/*
 * Block-sparse attention. The wmrh.cn FlashAttention v2 article (section 6,
 * future directions) suggests combining the method with block-sparse
 * patterns; the page fixes no format, so this one is:
 *   - the sequence is cut into blocks of FA2_BLOCKSPARSE_BLOCK = 128
 *     positions, nb = ceil(N / 128) per side;
 *   - block_mask: DEVICE bytes; the byte of (batch b, head h, query block r,
 *     key block c) is block_mask[b * mask_stride_b + h * mask_stride_h +
 *     r * nb + c] (strides in bytes, >= 0; 0 shares one mask across batches or
 *     heads). Non-zero: the block pair is computed; zero: it is skipped;
 *   - key j is visible to query i iff the dense rule (causal, window) allows
 *     it AND the byte of (i / 128, j / 128) is non-zero; ALiBi is unchanged;
 *   - a query row left with no visible key gets O = 0, LSE = -inf and zero
 *     gradients (its dO contributes nothing).
 * Skipped blocks cost neither memory traffic nor matrix work: each workgroup
 * compacts the tiles of its active blocks and streams only those.
 * Layouts, other arguments and errors as for fa2_fwd / fa2_bwd. N above 65536
 * is FA2_ERR_UNSUPPORTED; a null block_mask or a negative stride is
 * FA2_ERR_INVALID_ARG. The backward is always the atomic-free algorithm
 * (bitwise repeatable) and needs 2 * round_up(4 * B * H * N, 256) workspace
 * bytes.
 */
#define FA2_BLOCKSPARSE_BLOCK 128

fa2_status_t fa2_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse,
                                 int B, int H, int N, int d, float softmax_scale, int causal,
                                 int window_left, int window_right, const float* alibi_slopes,
                                 const unsigned char* block_mask, long long mask_stride_b,
                                 long long mask_stride_h, void* stream);

fa2_status_t fa2_bwd_blocksparse(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                 void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                                 float softmax_scale, int causal, int window_left, int window_right,
                                 const float* alibi_slopes, const unsigned char* block_mask,
                                 long long mask_stride_b, long long mask_stride_h, void* stream);

/*
 * Dropout on the attention weights. The wmrh.cn FlashAttention v2 article
 * (section 5.1, API) lists a dropout_p argument; the page fixes no random
 * number generator, so the keep matrix is defined here:
 *   - weight (i, j) of batch b, head h is kept iff v < keep, where v is an
 *     8-bit value of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 *     random numbers: as easy as 1, 2, 3", SC 2011) with key
 *     (seed mod 2^32, seed div 2^32) and counter (j / 16, i, b * H + h,
 *     offset): the call's four 32-bit words hold sixteen 8-bit values, value
 *     j % 16 at bits 8 * (j % 4) of word (j % 16) / 4;
 *     keep = floor((1 - dropout_p) * 256 + 0.5) (dropout_p as a float, the
 *     product in double), so the keep probability keep / 256 resolves
 *     dropout_p to 1/256;
 *   - O = (P * Z) V / (1 - dropout_p) with P the softmax of the dense
 *     definition (masks and ALiBi as for fa2_fwd); lse is that of the undropped
 *     softmax, so the backward rebuilds P from it as usual;
 *   - the backward regenerates Z from the same seed and offset:
 *     dV = (P * Z)^T dO / (1 - p), dS = P * (Z * dP / (1 - p) - D), with
 *     D = rowsum(dO * O) and O the dropped output the forward wrote.
 * dropout_p must be in [0, 1) and offset below 2^32 (else
 * FA2_ERR_INVALID_ARG); dropout_p = 0 is the dense
 * computation. Distinct (seed, offset) pairs give independent keep matrices;
 * callers advance `offset` between calls that share a seed. Layouts, other
 * arguments and errors as for fa2_fwd / fa2_bwd; the backward is the
 * atomic-free algorithm (bitwise repeatable) and needs
 * 2 * round_up(4 * B * H * N, 256) workspace bytes. Fixed-length dense batches
 * only (no packed or block-sparse variant).
 */
fa2_status_t fa2_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                             int B, int H, int N, int d, float softmax_scale, int causal,
                             int window_left, int window_right, const float* alibi_slopes,
                             float dropout_p, unsigned long long seed, unsigned long long offset,
                             void* stream);

fa2_status_t fa2_bwd_dropout(const void* q, const void* k, const void* v, const void* out,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                             float softmax_scale, int causal, int window_left, int window_right,
                             const float* alibi_slopes, float dropout_p, unsigned long long seed,
                             unsigned long long offset, void* stream);

/*
 * fa2_bwd without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments and results as fa2_bwd with deterministic = 1
 * (the atomic-free passes; bitwise the same gradients), minus workspace and
 * workspace_bytes. Its per-row scratch (8 bytes per row of B * H * N) lives in a
 * 16 MiB device array inside the library, one copy per GPU, held until the
 * process ends; nothing is allocated or freed by the call. Limit:
 * B * H * N <= 2^21 rows (e.g. B=4, H=32, N=16384), else FA2_ERR_UNSUPPORTED
 * before any HIP call. Calls that overlap on one GPU (other streams or host
 * threads) share the array and race: serialise them. Every byte it reads is
 * written earlier in the same call, so nothing needs clearing between calls.
 */
fa2_status_t fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int B, int H, int N, int d, float softmax_scale, int causal,
                             int window_left, int window_right, const float* alibi_slopes,
                             void* stream);

/* Static, human-readable name of a status code. */
const char* fa2_status_string(fa2_status_t status);

/* Library version as 10000*major + 100*minor + patch. */
int fa2_version(void);

/*
 * The window every entry point applies for a problem of n tokens (n = N, or
 * total_tokens for a packed batch): a side >= n - 1 already reaches every key
 * and is treated as -1 (unbounded), so windows up to INT_MAX behave like -1;
 * causal != 0 makes the right side 0. Writes the two values and returns FA2_OK;
 * FA2_ERR_INVALID_ARG for n < 0, a window < -1 or a null output pointer.
 * Host-only: touches no device and no stream. Source: window_size of section
 * 5.1 of the wmrh.cn FlashAttention v2 article (-1 = unbounded).
 */
fa2_status_t fa2_effective_window(int n, int causal, int window_left, int window_right,
                                  int* left_out, int* right_out);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
