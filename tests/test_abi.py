"""The C ABI on the CPU: the library loads, exports every function include/fa2.h
declares, and rejects bad arguments before any HIP call (nothing here launches)."""
import ctypes
import math
import os
import re

import pytest

import exact_tiled_attention_06_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

FAKE = 0x10000  # aligned, never dereferenced: every call below is rejected first
MISALIGNED = 0x10008


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa2.LIB_PATH):
        pytest.fail("libfa2.so is not built; run __graft_entry__.build()")
    return fa2.load_library()


def test_header_declares_the_documented_entry_points():
    assert header_functions() == sorted(
        ["fa2_fwd", "fa2_fwd_f32", "fa2_bwd", "fa2_bwd_workspace_size", "fa2_bwd_prep", "fa2_bwd_dkdv",
         "fa2_bwd_dq", "fa2_bwd_dq_stats", "fa2_fwd_varlen", "fa2_bwd_varlen", "fa2_fwd_blocksparse", "fa2_bwd_blocksparse",
         "fa2_fwd_dropout", "fa2_bwd_dropout", "fa2_status_string", "fa2_version", "fa2_effective_window",
         "fa2_bwd_noalloc"])


def test_library_exports_every_header_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(fa2.SIGNATURES) == set(header_functions())


def test_version_and_status_strings(lib):
    assert fa2.fa2_version() == 10000
    assert fa2.fa2_status_string(0) == "FA2_OK"
    for s in (1, 2, 3):
        assert fa2.fa2_status_string(s).startswith("FA2_ERR")
    assert "unknown" in fa2.fa2_status_string(99)


def fwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, B=1, H=2, N=16, d=64, scale=0.125,
             causal=0, wl=-1, wr=-1, alibi=None, stream=None)
    a.update(over)
    return [a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
            a["causal"], a["wl"], a["wr"], a["alibi"], a["stream"]]


BAD_FWD = [
    (dict(d=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(d=32), fa2.FA2_ERR_UNSUPPORTED),
    (dict(d=0), fa2.FA2_ERR_INVALID_ARG),
    (dict(B=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(H=-3), fa2.FA2_ERR_INVALID_ARG),
    (dict(N=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=0.0), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=math.inf), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=math.nan), fa2.FA2_ERR_INVALID_ARG),
    (dict(wl=-2), fa2.FA2_ERR_INVALID_ARG),
    (dict(wr=-7), fa2.FA2_ERR_INVALID_ARG),
    (dict(q=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(k=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(v=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(out=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(lse=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(q=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
    (dict(out=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
    (dict(alibi=FAKE + 2), fa2.FA2_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("fn", ["fa2_fwd", "fa2_fwd_f32"])
@pytest.mark.parametrize("over,status", BAD_FWD)
def test_forward_rejects_bad_arguments(lib, fn, over, status):
    assert getattr(lib, fn)(*fwd_args(**over)) == status


@pytest.mark.parametrize("fn", ["fa2_fwd", "fa2_fwd_f32"])
@pytest.mark.parametrize("over", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=None, out=None)])
def test_forward_empty_problem_is_ok_and_launches_nothing(lib, fn, over):
    assert getattr(lib, fn)(*fwd_args(**over)) == fa2.FA2_OK


def bwd_args(**over):
    a = dict(B=1, H=2, N=16, d=64)
    a.update({k: v for k, v in over.items() if k in a})
    ws = lib_ws = fa2.fa2_bwd_workspace_size(a["B"], a["H"], a["N"], a["d"])
    b = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             ws=FAKE, ws_bytes=max(ws, 0), scale=0.125, causal=1, wl=-1, wr=-1, alibi=None, det=0,
             stream=None)
    b.update({k: v for k, v in over.items() if k in b})
    del lib_ws
    return [b["q"], b["k"], b["v"], b["out"], b["lse"], b["dout"], b["dq"], b["dk"], b["dv"], b["ws"],
            b["ws_bytes"], a["B"], a["H"], a["N"], a["d"], b["scale"], b["causal"], b["wl"], b["wr"],
            b["alibi"], b["det"], b["stream"]]


BAD_BWD = [
    (dict(d=80), fa2.FA2_ERR_UNSUPPORTED),
    (dict(N=-4), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=0.0), fa2.FA2_ERR_INVALID_ARG),
    (dict(wl=-5), fa2.FA2_ERR_INVALID_ARG),
    (dict(dout=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(dq=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(dk=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws_bytes=100), fa2.FA2_ERR_INVALID_ARG),
    (dict(ws=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
    (dict(alibi=FAKE + 1), fa2.FA2_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("over,status", BAD_BWD)
def test_backward_rejects_bad_arguments(lib, over, status):
    assert lib.fa2_bwd(*bwd_args(**over)) == status


def test_backward_empty_problem_is_ok(lib):
    assert lib.fa2_bwd(*bwd_args(B=0, ws=None, ws_bytes=0)) == fa2.FA2_OK


def test_pass_entry_points_reject_bad_arguments(lib):
    ws = 512
    # prep: null dout, null lse, bad d, bad scale, too-small workspace
    assert lib.fa2_bwd_prep(FAKE, None, FAKE, FAKE, ws, 1, 2, 16, 64, 0.125, None) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_prep(FAKE, FAKE, None, FAKE, ws, 1, 2, 16, 64, 0.125, None) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_prep(FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 16, 96, 0.125, None) == fa2.FA2_ERR_UNSUPPORTED
    assert lib.fa2_bwd_prep(FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 16, 64, 0.0, None) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_prep(FAKE, FAKE, FAKE, FAKE, 256, 1, 2, 16, 64, 0.125, None) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_prep(FAKE, FAKE, FAKE, FAKE, ws, 0, 2, 16, 64, 0.125, None) == fa2.FA2_OK
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 16, 64, 0.125, 1, -1, -1, None, None]
    assert lib.fa2_bwd_dkdv(*args[:5], None, *args[6:]) == fa2.FA2_ERR_INVALID_ARG          # dk null
    assert lib.fa2_bwd_dkdv(*args[:13], 0.0, *args[14:]) == fa2.FA2_ERR_INVALID_ARG         # scale
    assert lib.fa2_bwd_dkdv(*args[:8], 4, *args[9:]) == fa2.FA2_ERR_INVALID_ARG            # workspace
    dq_args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 16, 64, 0.125, 1, -1, -1, None, None]
    assert lib.fa2_bwd_dq(*dq_args[:5], None, *dq_args[6:]) == fa2.FA2_ERR_INVALID_ARG      # dq null
    assert lib.fa2_bwd_dq(*dq_args[:14], -3, *dq_args[15:]) == fa2.FA2_ERR_INVALID_ARG     # window
    assert lib.fa2_bwd_dq(*dq_args[:11], 128 + 1, *dq_args[12:]) == fa2.FA2_ERR_UNSUPPORTED
    st_args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 1, 2, 16, 64, 0.125, 1, -1, -1, None, None]
    assert lib.fa2_bwd_dq_stats(*st_args[:3], None, *st_args[4:]) == fa2.FA2_ERR_INVALID_ARG  # out null
    assert lib.fa2_bwd_dq_stats(*st_args[:3], MISALIGNED, *st_args[4:]) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_dq_stats(*st_args[:8], 4, *st_args[9:]) == fa2.FA2_ERR_INVALID_ARG  # workspace
    assert lib.fa2_bwd_dq_stats(*st_args[:12], 96, *st_args[13:]) == fa2.FA2_ERR_UNSUPPORTED
    assert lib.fa2_bwd_dq_stats(*st_args[:9], 0, *st_args[10:]) == fa2.FA2_OK  # empty


def varlen_fwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, cu=FAKE, B=3, T=100, H=2, d=64, scale=0.125, causal=1,
             wl=-1, wr=-1, alibi=None, stream=None)
    a.update(over)
    return [a["q"], a["k"], a["v"], a["out"], a["lse"], a["cu"], a["B"], a["T"], a["H"], a["d"], a["scale"],
            a["causal"], a["wl"], a["wr"], a["alibi"], a["stream"]]


def varlen_bwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, cu=FAKE, ws=FAKE,
             ws_bytes=2048, B=3, T=100, H=2, d=64, scale=0.125, causal=1, wl=-1, wr=-1, alibi=None, stream=None)
    a.update(over)
    return [a[k] for k in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "cu", "ws", "ws_bytes", "B", "T",
                           "H", "d", "scale", "causal", "wl", "wr", "alibi", "stream")]


BAD_VARLEN = [
    (dict(cu=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(cu=FAKE + 2), fa2.FA2_ERR_INVALID_ARG),
    (dict(B=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(T=-5), fa2.FA2_ERR_INVALID_ARG),
    (dict(B=0), fa2.FA2_ERR_INVALID_ARG),          # tokens but no sequence
    (dict(d=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(scale=0.0), fa2.FA2_ERR_INVALID_ARG),
    (dict(wl=-3), fa2.FA2_ERR_INVALID_ARG),
    (dict(q=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(lse=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
    (dict(alibi=FAKE + 1), fa2.FA2_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("over,status", BAD_VARLEN)
def test_varlen_entry_points_reject_bad_arguments(lib, over, status):
    assert lib.fa2_fwd_varlen(*varlen_fwd_args(**over)) == status
    assert lib.fa2_bwd_varlen(*varlen_bwd_args(**over)) == status


def test_varlen_backward_checks_workspace_and_gradients(lib):
    need = fa2.fa2_bwd_workspace_size(1, 2, 100, 64)
    assert need >= 2 * 1024  # -D and -LSE / scale: 2 * 100 floats each, rounded up to 256 bytes
    assert lib.fa2_bwd_varlen(*varlen_bwd_args(ws_bytes=2 * 1024 - 4)) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_varlen(*varlen_bwd_args(dk=None)) == fa2.FA2_ERR_INVALID_ARG
    assert lib.fa2_bwd_varlen(*varlen_bwd_args(dout=MISALIGNED)) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("over", [dict(T=0), dict(B=0, T=0), dict(H=0), dict(T=0, cu=None, q=None)])
def test_varlen_empty_problem_is_ok_and_launches_nothing(lib, over):
    assert lib.fa2_fwd_varlen(*varlen_fwd_args(**over)) == fa2.FA2_OK
    assert lib.fa2_bwd_varlen(*varlen_bwd_args(**over)) == fa2.FA2_OK


def sparse_args(fn, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE,
             ws_bytes=8192, B=1, H=2, N=300, d=64, scale=0.125, causal=1, wl=-1, wr=-1, alibi=None, mask=FAKE,
             sb=0, sh=9, stream=None)
    a.update(over)
    if fn == "fa2_fwd_blocksparse":
        keys = ("q", "k", "v", "out", "lse", "B", "H", "N", "d", "scale", "causal", "wl", "wr", "alibi", "mask", "sb",
                "sh", "stream")
    else:
        keys = ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "ws", "ws_bytes", "B", "H", "N", "d", "scale",
                "causal", "wl", "wr", "alibi", "mask", "sb", "sh", "stream")
    return [a[k] for k in keys]


BAD_SPARSE = [
    (dict(mask=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(sb=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(sh=-9), fa2.FA2_ERR_INVALID_ARG),
    (dict(N=65537), fa2.FA2_ERR_UNSUPPORTED),
    (dict(d=80), fa2.FA2_ERR_UNSUPPORTED),
    (dict(N=-2), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=math.nan), fa2.FA2_ERR_INVALID_ARG),
    (dict(q=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(out=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("fn", ["fa2_fwd_blocksparse", "fa2_bwd_blocksparse"])
@pytest.mark.parametrize("over,status", BAD_SPARSE)
def test_blocksparse_entry_points_reject_bad_arguments(lib, fn, over, status):
    assert getattr(lib, fn)(*sparse_args(fn, **over)) == status


@pytest.mark.parametrize("fn", ["fa2_fwd_blocksparse", "fa2_bwd_blocksparse"])
def test_blocksparse_empty_problem_is_ok(lib, fn):
    assert getattr(lib, fn)(*sparse_args(fn, B=0, mask=None)) == fa2.FA2_OK


def test_blocksparse_backward_checks_workspace(lib):
    args = sparse_args("fa2_bwd_blocksparse", ws_bytes=2 * 2560 - 1)
    assert lib.fa2_bwd_blocksparse(*args) == fa2.FA2_ERR_INVALID_ARG


def dropout_args(fn, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE,
             ws_bytes=8192, B=1, H=2, N=300, d=128, scale=0.125, causal=1, wl=-1, wr=-1, alibi=None, p=0.1,
             seed=1, offset=2, stream=None)
    a.update(over)
    if fn == "fa2_fwd_dropout":
        keys = ("q", "k", "v", "out", "lse", "B", "H", "N", "d", "scale", "causal", "wl", "wr", "alibi", "p", "seed",
                "offset", "stream")
    else:
        keys = ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "ws", "ws_bytes", "B", "H", "N", "d", "scale",
                "causal", "wl", "wr", "alibi", "p", "seed", "offset", "stream")
    return [a[k] for k in keys]


BAD_DROPOUT = [
    (dict(p=1.0), fa2.FA2_ERR_INVALID_ARG),
    (dict(p=-0.25), fa2.FA2_ERR_INVALID_ARG),
    (dict(p=math.nan), fa2.FA2_ERR_INVALID_ARG),
    (dict(p=math.inf), fa2.FA2_ERR_INVALID_ARG),
    (dict(d=96), fa2.FA2_ERR_UNSUPPORTED),
    (dict(N=-1), fa2.FA2_ERR_INVALID_ARG),
    (dict(wl=-2), fa2.FA2_ERR_INVALID_ARG),
    (dict(scale=0.0), fa2.FA2_ERR_INVALID_ARG),
    (dict(v=None), fa2.FA2_ERR_INVALID_ARG),
    (dict(lse=MISALIGNED), fa2.FA2_ERR_INVALID_ARG),
    (dict(offset=2**32), fa2.FA2_ERR_INVALID_ARG),  # the generator's counter word is 32 bits
    (dict(offset=2**64 - 1), fa2.FA2_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("fn", ["fa2_fwd_dropout", "fa2_bwd_dropout"])
@pytest.mark.parametrize("over,status", BAD_DROPOUT)
def test_dropout_entry_points_reject_bad_arguments(lib, fn, over, status):
    assert getattr(lib, fn)(*dropout_args(fn, **over)) == status


@pytest.mark.parametrize("fn", ["fa2_fwd_dropout", "fa2_bwd_dropout"])
def test_dropout_empty_problem_is_ok(lib, fn):
    assert getattr(lib, fn)(*dropout_args(fn, H=0, q=None)) == fa2.FA2_OK
    # an invalid rate is still rejected on an empty problem
    assert getattr(lib, fn)(*dropout_args(fn, H=0, p=1.5)) == fa2.FA2_ERR_INVALID_ARG
    assert getattr(lib, fn)(*dropout_args(fn, H=0, offset=2**32)) == fa2.FA2_ERR_INVALID_ARG
    assert getattr(lib, fn)(*dropout_args(fn, H=0, offset=2**32 - 1, seed=2**64 - 1)) == fa2.FA2_OK


def test_dropout_backward_checks_workspace(lib):
    args = dropout_args("fa2_bwd_dropout", ws_bytes=2 * 2560 - 1)
    assert lib.fa2_bwd_dropout(*args) == fa2.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", ["fa2_fwd", "fa2_fwd_f32"])
def test_forward_rejects_too_many_heads_for_32_bit_tile_offsets(lib, fn):
    # H * d > 2^22: a 256-row tile would span 4 GiB or more
    assert getattr(lib, fn)(*fwd_args(H=32769, d=128)) == fa2.FA2_ERR_UNSUPPORTED
    assert getattr(lib, fn)(*fwd_args(H=65537, d=64)) == fa2.FA2_ERR_UNSUPPORTED


def test_workspace_size(lib):
    # -D and -LSE / scale [B,H,N] + float32 dQ accumulator [B,H,N,d], each rounded up to 256 bytes
    B, H, N, d = 4, 16, 4096, 128
    rows = B * H * N
    up = lambda x: (x + 255) // 256 * 256
    assert fa2.fa2_bwd_workspace_size(B, H, N, d) == up(rows * d * 4) + 2 * up(rows * 4)
    assert fa2.fa2_bwd_workspace_size(1, 1, 17, 64) == up(17 * 64 * 4) + 2 * up(17 * 4)
    assert fa2.fa2_bwd_workspace_size(0, 1, 17, 64) == 0
    assert fa2.fa2_bwd_workspace_size(1, 1, 17, 96) == 0


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(fa2.FA2Error):
        fa2.load_library(str(tmp_path / "absent.so"))


def test_product_package_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "exact_tiled_attention_06_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower().replace("no oracle", ""), f


def test_wrapper_workspace_for_the_atomic_free_backward(lib, monkeypatch):
    # -D and -LSE / scale only: the library's size minus the float32 dQ accumulator
    up = lambda x: (x + 255) // 256 * 256
    for B, H, N, d in [(4, 32, 8192, 128), (1, 3, 77, 64), (2, 1, 1, 128)]:
        rows = B * H * N
        assert fa2._split_workspace_bytes(rows) == fa2.fa2_bwd_workspace_size(B, H, N, d) - up(rows * d * 4)
    monkeypatch.delenv("FA2_BWD_ATOMIC_DQ", raising=False)
    assert not fa2._atomic_dq_selected(False)
    monkeypatch.setenv("FA2_BWD_ATOMIC_DQ", "1")
    assert fa2._atomic_dq_selected(False) and not fa2._atomic_dq_selected(True)


INT_MAX = 2**31 - 1


@pytest.mark.parametrize("n, causal, wl, wr, want", [
    (100, 0, -1, -1, (-1, -1)),
    (100, 0, 37, 5, (37, 5)),
    (100, 0, 98, 98, (98, 98)),        # below n - 1: kept
    (100, 0, 99, 99, (-1, -1)),        # n - 1 reaches every key
    (100, 0, INT_MAX, INT_MAX, (-1, -1)),
    (100, 1, INT_MAX, INT_MAX, (-1, 0)),  # causal: right side 0
    (100, 1, 50, -1, (50, 0)),
    (1, 0, 0, 0, (-1, -1)),            # a single token: every window reaches it
    (0, 0, 5, 5, (-1, -1)),
])
def test_effective_window(lib, n, causal, wl, wr, want):
    assert fa2.fa2_effective_window(n, causal, wl, wr) == want


@pytest.mark.parametrize("args", [(-1, 0, -1, -1), (10, 0, -2, -1), (10, 0, -1, -2)])
def test_effective_window_rejects(lib, args):
    with pytest.raises(fa2.FA2Error):
        fa2.fa2_effective_window(*args)


def test_huge_n_is_unsupported(lib):
    st = lib.fa2_fwd(*fwd_args(N=(1 << 30) + 1, B=1, H=1))
    assert st == fa2.FA2_ERR_UNSUPPORTED


def test_grid_beyond_a_signed_32_bit_workgroup_id_is_unsupported(lib):
    # 2^24 blocks of 64 rows per head times 129 heads: 2^31 + 2^24 workgroups
    assert lib.fa2_fwd(*fwd_args(N=1 << 30, B=129, H=1, d=64)) == fa2.FA2_ERR_UNSUPPORTED


def test_noalloc_backward_rejects_before_any_hip_call(lib):
    """Too many rows for its scratch array, and invalid arguments, are rejected before any
    HIP call (so on a machine without a GPU too)."""
    def call(B, H, N, d=128, q=FAKE, scale=0.125):
        return lib.fa2_bwd_noalloc(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, H, N, d, scale, 1, -1, -1,
                                   None, None)
    assert call(4, 32, 16384 + 1) == fa2.FA2_ERR_UNSUPPORTED   # 2^21 + 128 rows
    assert call(1, 1, (1 << 21) + 1) == fa2.FA2_ERR_UNSUPPORTED
    assert call(1, 1, 64, d=96) == fa2.FA2_ERR_UNSUPPORTED
    assert call(1, 1, 64, q=None) == fa2.FA2_ERR_INVALID_ARG
    assert call(1, 1, 64, q=MISALIGNED) == fa2.FA2_ERR_INVALID_ARG
    assert call(1, 1, 64, scale=0.0) == fa2.FA2_ERR_INVALID_ARG
    assert call(0, 1, 64) == fa2.FA2_OK                        # empty problem
