"""Python binding of libfa2.so, the MI355X exact-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa2.h. PyTorch supplies device
memory and the current stream. If the library has not been built, every call
raises FA2Error; there is no fallback path.

Low-level functions carry the C names and arguments (fa2_fwd, fa2_fwd_f32,
fa2_bwd, fa2_bwd_workspace_size, fa2_bwd_prep, fa2_bwd_dkdv, fa2_bwd_dq,
fa2_fwd_varlen, fa2_bwd_varlen, fa2_fwd_blocksparse, fa2_bwd_blocksparse,
fa2_fwd_dropout, fa2_bwd_dropout, fa2_status_string, fa2_version); tensors or
raw device addresses (int) are accepted for pointers. The convenience
functions ``flash_attn_fwd`` / ``flash_attn_bwd`` mirror the parameter list of
the FlashAttention v2 API on the wmrh.cn article (section 5.1):
dropout_p=0.0 (with seed and offset for its keep matrix), softmax_scale=None
(-> 1/sqrt(d)), causal, window_size=(-1, -1), alibi_slopes, and deterministic
for the backward. ``flash_attn_varlen_fwd`` /
``flash_attn_varlen_bwd`` take sequences packed as [T, H, d] with int32
boundaries ``cu_seqlens`` [B + 1] (variable-length batches, section 6 of the
same article). ``flash_attn_blocksparse_fwd`` / ``flash_attn_blocksparse_bwd``
take a uint8 block mask over 128 x 128 blocks (block-sparse patterns, also
section 6).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA2Error", "LIB_PATH", "load_library", "fa2_fwd", "fa2_fwd_f32", "fa2_bwd",
    "fa2_bwd_workspace_size", "fa2_bwd_prep", "fa2_bwd_dkdv", "fa2_bwd_dq", "fa2_bwd_dq_stats", "fa2_fwd_varlen", "fa2_bwd_varlen",
    "fa2_fwd_blocksparse", "fa2_bwd_blocksparse", "fa2_fwd_dropout", "fa2_bwd_dropout", "fa2_status_string", "fa2_version", "fa2_effective_window", "fa2_bwd_noalloc", "flash_attn_fwd",
    "flash_attn_bwd", "flash_attn_varlen_fwd", "flash_attn_varlen_bwd", "flash_attn_blocksparse_fwd",
    "flash_attn_blocksparse_bwd", "BLOCKSPARSE_BLOCK", "FA2_OK", "FA2_ERR_INVALID_ARG", "FA2_ERR_UNSUPPORTED", "FA2_ERR_HIP",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa2.so")

BLOCKSPARSE_BLOCK = 128  # FA2_BLOCKSPARSE_BLOCK

FA2_OK = 0
FA2_ERR_INVALID_ARG = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_HIP = 3

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_L = ctypes.c_longlong
_U64 = ctypes.c_ulonglong

# C signatures of include/fa2.h
SIGNATURES = {
    "fa2_fwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P], _I),
    "fa2_fwd_f32": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P], _I),
    "fa2_bwd_workspace_size": ([_I, _I, _I, _I], ctypes.c_size_t),
    "fa2_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I,
                 _P, _I, _P], _I),
    "fa2_bwd_prep": ([_P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _P], _I),
    "fa2_bwd_dkdv": ([_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P], _I),
    "fa2_bwd_dq": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P], _I),
    "fa2_bwd_dq_stats": ([_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P],
                         _I),
    "fa2_fwd_varlen": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P], _I),
    "fa2_bwd_varlen": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I,
                        _P, _P], _I),
    "fa2_fwd_blocksparse": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P, _L, _L, _P], _I),
    "fa2_bwd_blocksparse": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I,
                             _P, _P, _L, _L, _P], _I),
    "fa2_fwd_dropout": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _F, _U64, _U64, _P], _I),
    "fa2_bwd_dropout": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _F, _I, _I, _I,
                         _P, _F, _U64, _U64, _P], _I),
    "fa2_status_string": ([_I], ctypes.c_char_p),
    "fa2_version": ([], _I),
    "fa2_bwd_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P], _I),
    "fa2_effective_window": ([_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)], _I),
}


class FA2Error(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def load_library(path: str | None = None):
    """Load libfa2.so (once). Raises FA2Error if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FA2Error(f"HIP library not built: {p} (run __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != FA2_OK:
        raise FA2Error(f"{what}: {fa2_status_string(status)}", status)


def fa2_status_string(status: int) -> str:
    s = load_library().fa2_status_string(int(status))
    return s.decode() if s else "unknown"


def fa2_version() -> int:
    return int(load_library().fa2_version())


def fa2_bwd_noalloc(q, k, v, out, lse, dout, dq, dk, dv, B, H, N, d, softmax_scale, causal, window_left,
                    window_right, alibi_slopes=None, stream=None):
    st = load_library().fa2_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), int(B), int(H), int(N), int(d), float(softmax_scale),
                                        int(causal), int(window_left), int(window_right), _ptr(alibi_slopes),
                                        _stream(stream))
    _check(st, "fa2_bwd_noalloc")


def fa2_effective_window(n, causal, window_left, window_right):
    """(left, right) window the library applies for n tokens (host-only, no GPU)."""
    left, right = _I(0), _I(0)
    st = load_library().fa2_effective_window(int(n), int(causal), int(window_left), int(window_right),
                                             ctypes.byref(left), ctypes.byref(right))
    _check(st, "fa2_effective_window")
    return left.value, right.value


def fa2_fwd(q, k, v, out, lse, B, H, N, d, softmax_scale, causal, window_left, window_right,
            alibi_slopes=None, stream=None):
    st = load_library().fa2_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(N),
                                int(d), float(softmax_scale), int(causal), int(window_left),
                                int(window_right), _ptr(alibi_slopes), _stream(stream))
    _check(st, "fa2_fwd")


def fa2_fwd_f32(q, k, v, out, lse, B, H, N, d, softmax_scale, causal, window_left, window_right,
                alibi_slopes=None, stream=None):
    st = load_library().fa2_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H),
                                    int(N), int(d), float(softmax_scale), int(causal), int(window_left),
                                    int(window_right), _ptr(alibi_slopes), _stream(stream))
    _check(st, "fa2_fwd_f32")


def fa2_bwd_workspace_size(B, H, N, d) -> int:
    return int(load_library().fa2_bwd_workspace_size(int(B), int(H), int(N), int(d)))


def fa2_bwd(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, softmax_scale,
            causal, window_left, window_right, alibi_slopes=None, deterministic=0, stream=None):
    st = load_library().fa2_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace_bytes), int(B), int(H),
                                int(N), int(d), float(softmax_scale), int(causal), int(window_left),
                                int(window_right), _ptr(alibi_slopes), int(deterministic),
                                _stream(stream))
    _check(st, "fa2_bwd")


def fa2_bwd_prep(out, dout, lse, workspace, workspace_bytes, B, H, N, d, softmax_scale, stream=None):
    st = load_library().fa2_bwd_prep(_ptr(out), _ptr(dout), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                     int(B), int(H), int(N), int(d), float(softmax_scale), _stream(stream))
    _check(st, "fa2_bwd_prep")


def fa2_bwd_dkdv(q, k, v, lse, dout, dk, dv, workspace, workspace_bytes, B, H, N, d, softmax_scale, causal,
                 window_left, window_right, alibi_slopes=None, stream=None):
    st = load_library().fa2_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dk), _ptr(dv),
                                     _ptr(workspace), int(workspace_bytes), int(B), int(H), int(N), int(d),
                                     float(softmax_scale), int(causal), int(window_left), int(window_right),
                                     _ptr(alibi_slopes), _stream(stream))
    _check(st, "fa2_bwd_dkdv")


def fa2_bwd_dq(q, k, v, lse, dout, dq, workspace, workspace_bytes, B, H, N, d, softmax_scale, causal,
               window_left, window_right, alibi_slopes=None, stream=None):
    st = load_library().fa2_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(workspace),
                                   int(workspace_bytes), int(B), int(H), int(N), int(d), float(softmax_scale),
                                   int(causal), int(window_left), int(window_right), _ptr(alibi_slopes),
                                   _stream(stream))
    _check(st, "fa2_bwd_dq")


def fa2_bwd_dq_stats(q, k, v, out, lse, dout, dq, workspace, workspace_bytes, B, H, N, d, softmax_scale, causal,
                     window_left, window_right, alibi_slopes=None, stream=None):
    st = load_library().fa2_bwd_dq_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                         _ptr(workspace), int(workspace_bytes), int(B), int(H), int(N), int(d),
                                         float(softmax_scale), int(causal), int(window_left), int(window_right),
                                         _ptr(alibi_slopes), _stream(stream))
    _check(st, "fa2_bwd_dq_stats")


def fa2_fwd_varlen(q, k, v, out, lse, cu_seqlens, B, total_tokens, H, d, softmax_scale, causal, window_left,
                   window_right, alibi_slopes=None, stream=None):
    st = load_library().fa2_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), int(B),
                                       int(total_tokens), int(H), int(d), float(softmax_scale), int(causal),
                                       int(window_left), int(window_right), _ptr(alibi_slopes), _stream(stream))
    _check(st, "fa2_fwd_varlen")


def fa2_bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, cu_seqlens, workspace, workspace_bytes, B, total_tokens, H,
                   d, softmax_scale, causal, window_left, window_right, alibi_slopes=None, stream=None):
    st = load_library().fa2_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(cu_seqlens), _ptr(workspace), int(workspace_bytes),
                                       int(B), int(total_tokens), int(H), int(d), float(softmax_scale), int(causal),
                                       int(window_left), int(window_right), _ptr(alibi_slopes), _stream(stream))
    _check(st, "fa2_bwd_varlen")


def fa2_fwd_blocksparse(q, k, v, out, lse, B, H, N, d, softmax_scale, causal, window_left, window_right,
                        alibi_slopes, block_mask, mask_stride_b, mask_stride_h, stream=None):
    st = load_library().fa2_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(N),
                                            int(d), float(softmax_scale), int(causal), int(window_left),
                                            int(window_right), _ptr(alibi_slopes), _ptr(block_mask),
                                            int(mask_stride_b), int(mask_stride_h), _stream(stream))
    _check(st, "fa2_fwd_blocksparse")


def fa2_bwd_blocksparse(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, softmax_scale,
                        causal, window_left, window_right, alibi_slopes, block_mask, mask_stride_b, mask_stride_h,
                        stream=None):
    st = load_library().fa2_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                            _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace_bytes), int(B), int(H),
                                            int(N), int(d), float(softmax_scale), int(causal), int(window_left),
                                            int(window_right), _ptr(alibi_slopes), _ptr(block_mask),
                                            int(mask_stride_b), int(mask_stride_h), _stream(stream))
    _check(st, "fa2_bwd_blocksparse")


def fa2_fwd_dropout(q, k, v, out, lse, B, H, N, d, softmax_scale, causal, window_left, window_right,
                    alibi_slopes, dropout_p, seed, offset, stream=None):
    st = load_library().fa2_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(B), int(H), int(N),
                                        int(d), float(softmax_scale), int(causal), int(window_left),
                                        int(window_right), _ptr(alibi_slopes), float(dropout_p), int(seed),
                                        int(offset), _stream(stream))
    _check(st, "fa2_fwd_dropout")


def fa2_bwd_dropout(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, softmax_scale,
                    causal, window_left, window_right, alibi_slopes, dropout_p, seed, offset, stream=None):
    st = load_library().fa2_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace_bytes), int(B), int(H),
                                        int(N), int(d), float(softmax_scale), int(causal), int(window_left),
                                        int(window_right), _ptr(alibi_slopes), float(dropout_p), int(seed),
                                        int(offset), _stream(stream))
    _check(st, "fa2_bwd_dropout")


# ------------------------------------------------------------------ convenience wrappers

def _check_tensors(*ts):
    import torch
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise FA2Error("expected torch tensors")
        if not t.is_cuda or t.device != ref.device:
            raise FA2Error("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise FA2Error("tensors must be contiguous [B, N, H, d]")
        if t.dtype != ref.dtype or t.shape != ref.shape:
            raise FA2Error("q, k, v (and out, dout) must share dtype and shape")


def _check_aux(lse, shape, device, workspace=None):
    """The forward's lse (float32, contiguous, the given shape, on the tensors' GPU)
    and, if given, a caller's workspace (on the same GPU): the kernels index them
    by position, so a wrong layout would read the wrong rows."""
    import torch
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32:
        raise FA2Error("lse must be a float32 tensor (the forward's output)")
    if tuple(lse.shape) != tuple(shape) or not lse.is_contiguous():
        raise FA2Error(f"lse must be contiguous with shape {tuple(shape)}, got {tuple(lse.shape)}")
    if lse.device != device:
        raise FA2Error("lse must be on the tensors' GPU")
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
            raise FA2Error("workspace must be a contiguous tensor on the tensors' GPU")


def _slopes(alibi_slopes, H, device):
    import torch
    if alibi_slopes is None:
        return None
    s = alibi_slopes.to(device=device, dtype=torch.float32).contiguous()
    if s.numel() != H:
        raise FA2Error("alibi_slopes must have H entries")
    return s


def flash_attn_fwd(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1), alibi_slopes=None,
                   dropout_p=0.0, seed=0, offset=0):
    """Exact attention forward. q, k, v: [B, N, H, d] bf16 or float32 on the GPU.
    dropout_p > 0 (bf16 only) drops attention weights with the keep matrix of
    (seed, offset) (see fa2_fwd_dropout in include/fa2.h).
    Returns (out [B, N, H, d], lse [B, H, N] float32, natural log)."""
    import torch
    _check_tensors(q, k, v)
    B, N, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    sl = _slopes(alibi_slopes, H, q.device)
    if dropout_p:
        if q.dtype != torch.bfloat16:
            raise FA2Error("dropout takes bf16 tensors")
        fa2_fwd_dropout(q, k, v, out, lse, B, H, N, d, scale, int(bool(causal)), window_size[0], window_size[1], sl,
                        dropout_p, seed, offset)
        return out, lse
    if q.dtype == torch.bfloat16:
        fn = fa2_fwd
    elif q.dtype == torch.float32:
        fn = fa2_fwd_f32
    else:
        raise FA2Error(f"unsupported dtype {q.dtype}")
    fn(q, k, v, out, lse, B, H, N, d, scale, int(bool(causal)), window_size[0], window_size[1], sl)
    return out, lse


def _split_workspace_bytes(rows):
    """Workspace of the atomic-free backward: -D and -LSE / scale, one float32 each per
    row, each array rounded up to 256 bytes (include/fa2.h)."""
    return max(2 * ((4 * rows + 255) // 256 * 256), 256)


def _atomic_dq_selected(deterministic):
    """fa2_bwd accumulates dQ atomically only when asked for no determinism and
    FA2_BWD_ATOMIC_DQ=1 is set; only that variant needs the float32 dQ accumulator."""
    return not deterministic and os.environ.get("FA2_BWD_ATOMIC_DQ") == "1"


def flash_attn_bwd(dout, q, k, v, out, lse, softmax_scale=None, causal=False, window_size=(-1, -1),
                   alibi_slopes=None, deterministic=False, workspace=None, dropout_p=0.0, seed=0, offset=0):
    """Exact attention backward from the forward's out and lse. bf16 [B, N, H, d] tensors.
    dropout_p, seed, offset must be those of the forward. Returns (dq, dk, dv)."""
    import torch
    _check_tensors(q, k, v, out, dout)
    if q.dtype != torch.bfloat16:
        raise FA2Error("the backward takes bf16 tensors")
    B, N, H, d = q.shape
    _check_aux(lse, (B, H, N), q.device, workspace)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        need = (fa2_bwd_workspace_size(B, H, N, d) if _atomic_dq_selected(deterministic) and not dropout_p
                else _split_workspace_bytes(B * H * N))
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sl = _slopes(alibi_slopes, H, q.device)
    if dropout_p:
        fa2_bwd_dropout(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace.numel() * workspace.element_size(),
                        B, H, N, d, scale, int(bool(causal)), window_size[0], window_size[1], sl, dropout_p, seed,
                        offset)
        return dq, dk, dv
    fa2_bwd(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace.numel() * workspace.element_size(),
            B, H, N, d, scale, int(bool(causal)), window_size[0], window_size[1], sl, int(bool(deterministic)))
    return dq, dk, dv


def _cu(cu_seqlens, device):
    import torch
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise FA2Error("cu_seqlens must be a 1-D int32 tensor [B + 1]")
    if cu_seqlens.device != device or not cu_seqlens.is_contiguous():
        raise FA2Error("cu_seqlens must be contiguous and on the tensors' GPU")
    return cu_seqlens


def flash_attn_varlen_fwd(q, k, v, cu_seqlens, softmax_scale=None, causal=False, window_size=(-1, -1),
                          alibi_slopes=None):
    """Packed variable-length forward. q, k, v: bf16 [T, H, d]; cu_seqlens: int32 [B + 1] on the GPU.
    Returns (out [T, H, d], lse [H, T] float32)."""
    import torch
    _check_tensors(q, k, v)
    if q.dtype != torch.bfloat16:
        raise FA2Error("packed batches take bf16 tensors")
    T, H, d = q.shape
    cu = _cu(cu_seqlens, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    fa2_fwd_varlen(q, k, v, out, lse, cu, cu.numel() - 1, T, H, d, scale, int(bool(causal)), window_size[0],
                   window_size[1], _slopes(alibi_slopes, H, q.device))
    return out, lse


def flash_attn_varlen_bwd(dout, q, k, v, out, lse, cu_seqlens, softmax_scale=None, causal=False,
                          window_size=(-1, -1), alibi_slopes=None, workspace=None):
    """Packed variable-length backward from the forward's out and lse. Returns (dq, dk, dv) [T, H, d]."""
    import torch
    _check_tensors(q, k, v, out, dout)
    if q.dtype != torch.bfloat16:
        raise FA2Error("packed batches take bf16 tensors")
    T, H, d = q.shape
    cu = _cu(cu_seqlens, q.device)
    _check_aux(lse, (H, T), q.device, workspace)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(_split_workspace_bytes(H * T), dtype=torch.uint8, device=q.device)
    fa2_bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, cu, workspace, workspace.numel() * workspace.element_size(),
                   cu.numel() - 1, T, H, d, scale, int(bool(causal)), window_size[0], window_size[1],
                   _slopes(alibi_slopes, H, q.device))
    return dq, dk, dv


def _block_mask(block_mask, B, H, N, device):
    """A uint8 mask [B or 1, H or 1, nb, nb] on the GPU -> (tensor, batch stride, head stride);
    a size-1 batch or head dimension is shared (stride 0)."""
    import torch
    nb = -(-N // BLOCKSPARSE_BLOCK)
    if not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8 or block_mask.dim() != 4:
        raise FA2Error("block_mask must be a 4-D uint8 tensor [B or 1, H or 1, nb, nb]")
    mb, mh, r, c = block_mask.shape
    if (r, c) != (nb, nb) or mb not in (1, B) or mh not in (1, H):
        raise FA2Error(f"block_mask shape {tuple(block_mask.shape)} does not fit B={B}, H={H}, nb={nb}")
    if block_mask.device != device or block_mask.stride(3) != 1 or block_mask.stride(2) != nb:
        raise FA2Error("block_mask must be on the tensors' GPU with contiguous [nb, nb] blocks")
    sb = block_mask.stride(0) if mb == B and B > 1 else 0
    sh = block_mask.stride(1) if mh == H and H > 1 else 0
    return block_mask, sb, sh


def flash_attn_blocksparse_fwd(q, k, v, block_mask, softmax_scale=None, causal=False, window_size=(-1, -1),
                               alibi_slopes=None):
    """Block-sparse forward. q, k, v: bf16 [B, N, H, d]; block_mask: uint8 [B or 1, H or 1, nb, nb]
    over 128 x 128 blocks (non-zero = computed). Returns (out, lse [B, H, N])."""
    import torch
    _check_tensors(q, k, v)
    if q.dtype != torch.bfloat16:
        raise FA2Error("block-sparse attention takes bf16 tensors")
    B, N, H, d = q.shape
    m, sb, sh = _block_mask(block_mask, B, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa2_fwd_blocksparse(q, k, v, out, lse, B, H, N, d, scale, int(bool(causal)), window_size[0], window_size[1],
                        _slopes(alibi_slopes, H, q.device), m, sb, sh)
    return out, lse


def flash_attn_blocksparse_bwd(dout, q, k, v, out, lse, block_mask, softmax_scale=None, causal=False,
                               window_size=(-1, -1), alibi_slopes=None, workspace=None):
    """Block-sparse backward from the forward's out and lse. Returns (dq, dk, dv)."""
    import torch
    _check_tensors(q, k, v, out, dout)
    if q.dtype != torch.bfloat16:
        raise FA2Error("block-sparse attention takes bf16 tensors")
    B, N, H, d = q.shape
    m, sb, sh = _block_mask(block_mask, B, H, N, q.device)
    _check_aux(lse, (B, H, N), q.device, workspace)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(_split_workspace_bytes(B * H * N), dtype=torch.uint8, device=q.device)
    fa2_bwd_blocksparse(q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace.numel() * workspace.element_size(),
                        B, H, N, d, scale, int(bool(causal)), window_size[0], window_size[1],
                        _slopes(alibi_slopes, H, q.device), m, sb, sh)
    return dq, dk, dv
