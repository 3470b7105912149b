"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic. It only draws inputs, so that the
HIP path, the fp64 oracle, the tests and the benchmark all see the same bytes.

Recipe (the same for every workload):
  * ``torch.Generator('cpu').manual_seed(seed)``; ``randn`` in float32, drawn in
    the order q, k, v, dout, each of shape ``[B, N, H, d]``;
  * bf16 workloads round those float32 draws to bf16 (round-to-nearest-even,
    ``Tensor.to(torch.bfloat16)``); both sides then read the same bf16 values;
  * ALiBi slopes, when a workload uses them, are ``2**(-8*(h+1)/H)`` for head
    ``h = 0..H-1``, stored as float32;
  * the default input seed is the workload number and the default
    row-sampling seed is ``1000 + number``.

Variable-length batches pack B sequences along the token axis ([T, H, d]
tensors, T = total tokens) with boundaries ``cu_seqlens`` ([B + 1] int32).
Their lengths come from B - 1 distinct cut points drawn uniformly from
1 .. T - 1 with ``numpy.random.default_rng(seed)``: a ragged mix of short and
long sequences (spacings of uniform cut points, mean T / B). The tensors are
drawn like a [1, T, H, d] batch and viewed as [T, H, d].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    dtype: str          # "f32" or "bf16": element type of q, k, v, out, dout, dq, dk, dv
    B: int
    H: int
    N: int
    d: int
    causal: bool
    window: tuple       # (window_left, window_right); -1 = unbounded
    alibi: bool
    backward: bool      # whether the workload includes the backward pass

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def shape(self):
        return (self.B, self.N, self.H, self.d)

    def describe(self) -> str:
        w = "" if self.window == (-1, -1) else f" window={self.window}"
        return (f"{self.name}: {self.dtype} B={self.B} H={self.H} N={self.N} d={self.d}"
                f" causal={int(self.causal)}{w} alibi={int(self.alibi)}")


WORKLOADS = {
    1: Workload(1, "tiny_f32_fwd", "f32", 1, 2, 128, 64, False, (-1, -1), False, False),
    2: Workload(2, "bf16_fwd_n2048_d64", "bf16", 8, 16, 2048, 64, False, (-1, -1), False, False),
    3: Workload(3, "bf16_causal_fwd_n8192_d128", "bf16", 4, 32, 8192, 128, True, (-1, -1), False, False),
    4: Workload(4, "bf16_causal_bwd_n4096_d128", "bf16", 4, 16, 4096, 128, True, (-1, -1), False, True),
    5: Workload(5, "bf16_window_alibi_n16384_d128", "bf16", 1, 32, 16384, 128, True, (4096, 0), True, True),
}


def alibi_slopes(H: int) -> torch.Tensor:
    """ALiBi slopes 2**(-8*(h+1)/H), h = 0..H-1, as float32 (an input, not a computation step)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def make_inputs(B, H, N, d, dtype="bf16", seed=0, with_dout=False):
    """Draw q, k, v (and dout) of shape [B, N, H, d] on the CPU, in the recipe above."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, N, H, d)
    names = ["q", "k", "v"] + (["dout"] if with_dout else [])
    out = {}
    for nm in names:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out[nm] = x if dtype == "f32" else x.to(torch.bfloat16)
    return out


def workload_inputs(w: Workload, seed=None, with_dout=None):
    """Inputs for a numbered workload, including ALiBi slopes (or None)."""
    seed = w.number if seed is None else seed
    with_dout = w.backward if with_dout is None else with_dout
    t = make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed, with_dout)
    t["alibi_slopes"] = alibi_slopes(w.H) if w.alibi else None
    return t


def sample_query_rows(B, H, N, count=256, seed=0):
    """`count` distinct (b, h, i) triples drawn uniformly with the seed, sorted."""
    rng = np.random.default_rng(seed)
    total = B * H * N
    count = min(count, total)
    flat = np.sort(rng.choice(total, size=count, replace=False))
    b = flat // (H * N)
    h = (flat // N) % H
    i = flat % N
    return np.stack([b, h, i], axis=1).astype(np.int64)


def sample_key_rows(B, H, N, count=256, max_heads=4, seed=0):
    """`count` distinct (b, h, j) key triples drawn from at most `max_heads` seeded heads."""
    rng = np.random.default_rng(seed + 7919)
    heads = rng.choice(B * H, size=min(max_heads, B * H), replace=False)
    per = max(1, count // len(heads))
    rows = []
    for bh in np.sort(heads):
        js = np.sort(rng.choice(N, size=min(per, N), replace=False))
        for j in js:
            rows.append((bh // H, bh % H, j))
    return np.array(rows, dtype=np.int64)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    number: int
    name: str
    dtype: str
    total: int          # packed tokens T
    nseq: int           # sequences B
    H: int
    d: int
    causal: bool
    window: tuple
    alibi: bool
    backward: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self) -> str:
        w = "" if self.window == (-1, -1) else f" window={self.window}"
        return (f"{self.name}: {self.dtype} T={self.total} B={self.nseq} H={self.H} d={self.d}"
                f" causal={int(self.causal)}{w} alibi={int(self.alibi)}")


# The same token budget and head shape as the causal N=8192 workload (4 x 8192
# tokens, H=32, d=128), split into 12 ragged sequences.
VARLEN_WORKLOADS = {
    6: VarlenWorkload(6, "bf16_varlen_causal_t32768_d128", "bf16", 32768, 12, 32, 128, True, (-1, -1), False, True),
}


def varlen_lengths(total: int, nseq: int, seed: int = 0) -> np.ndarray:
    """Lengths of nseq sequences (each >= 1) summing to total: spacings of nseq - 1
    distinct uniform cut points in 1 .. total - 1."""
    if nseq <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, total), size=nseq - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total]])
    return np.diff(edges).astype(np.int64)


def cu_seqlens_from_lengths(lengths) -> torch.Tensor:
    """Sequence boundaries [B + 1] int32: 0, then the running total of the lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))


def make_varlen_inputs(total, H, d, dtype="bf16", seed=0, with_dout=False):
    """Packed q, k, v (and dout) of shape [T, H, d], drawn like a [1, T, H, d] batch."""
    t = make_inputs(1, H, total, d, dtype, seed, with_dout)
    return {nm: x[0] for nm, x in t.items()}


def varlen_workload_inputs(w: VarlenWorkload, seed=None, with_dout=None):
    """Inputs of a variable-length workload: tensors, lengths, cu_seqlens and ALiBi slopes."""
    seed = w.number if seed is None else seed
    with_dout = w.backward if with_dout is None else with_dout
    t = make_varlen_inputs(w.total, w.H, w.d, w.dtype, seed, with_dout)
    t["lengths"] = varlen_lengths(w.total, w.nseq, seed)
    t["cu_seqlens"] = cu_seqlens_from_lengths(t["lengths"])
    t["alibi_slopes"] = alibi_slopes(w.H) if w.alibi else None
    return t


def sample_varlen_rows(total, H, count=256, seed=0):
    """`count` distinct (h, t) pairs (head, packed token) drawn uniformly with the seed, sorted."""
    rng = np.random.default_rng(seed)
    count = min(count, total * H)
    flat = np.sort(rng.choice(total * H, size=count, replace=False))
    return np.stack([flat // total, flat % total], axis=1).astype(np.int64)


# Block-sparse workload: the causal N=8192 shape with a 128 x 128 block mask.
@dataclasses.dataclass(frozen=True)
class BlockSparseWorkload:
    number: int
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    local: int          # key blocks r - local .. r are on (a band around the diagonal)
    global_blocks: int  # the first key blocks are on for every query block
    density: float      # every other block is on with this probability (seeded, per head)
    dtype: str = "bf16"
    window: tuple = (-1, -1)
    alibi: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def describe(self) -> str:
        return (f"{self.name}: bf16 B={self.B} H={self.H} N={self.N} d={self.d} causal={int(self.causal)} "
                f"mask: band {self.local}, {self.global_blocks} global, random {self.density}")


SPARSE_WORKLOADS = {
    7: BlockSparseWorkload(7, "bf16_blocksparse_causal_n8192_d128", 4, 32, 8192, 128, True, 1, 1, 0.1),
}


def sparse_block_mask(H, N, local=1, global_blocks=1, density=0.1, seed=0, block=128) -> torch.Tensor:
    """uint8 [1, H, nb, nb] block mask shared by every batch entry: for query block r,
    key blocks r - local .. r + local, the first `global_blocks` ones and a seeded
    random `density` share of the rest are on."""
    nb = -(-N // block)
    rng = np.random.default_rng(seed)
    m = (rng.random((H, nb, nb)) < density)
    r = np.arange(nb)[:, None]
    c = np.arange(nb)[None, :]
    m |= (np.abs(r - c) <= local)[None]
    m[:, :, :global_blocks] = True
    return torch.from_numpy(m.astype(np.uint8))[None]
