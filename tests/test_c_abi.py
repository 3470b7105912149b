"""The C ABI from a C program: tests/c/abi_check.c, compiled as C99 by the host C
compiler against include/fa2.h and linked with libfa2.so by name. Every call in it is
rejected by argument validation or is an empty problem, both of which return before
any HIP call, so it runs without a GPU and launches nothing."""
import os
import shutil
import subprocess

import pytest

import exact_tiled_attention_06_amd as fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_compiles_links_and_sees_the_documented_status_codes(tmp_path):
    if not os.path.exists(fa2.LIB_PATH):
        pytest.fail("libfa2.so is not built; run __graft_entry__.build()")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    libdir = os.path.dirname(fa2.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    build = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", libdir, "-l:libfa2.so",
                            f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True, timeout=120)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failure(s)" in run.stdout


def test_keep_mask_compare_matches_a_plain_byte_compare(tmp_path):
    """The dropout kernels' packed compare of generator bytes against the keep
    threshold (tests/c/keep_mask_check.cpp), built for the host only from the
    kernels' own header: every threshold, byte position and byte value."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc")
    exe = str(tmp_path / "keep_mask_check")
    build = subprocess.run([hipcc, "--cuda-host-only", "-O2", "-std=c++17", "-I",
                            os.path.join(ROOT, "exact_tiled_attention_06_amd", "csrc"),
                            os.path.join(ROOT, "tests", "c", "keep_mask_check.cpp"), "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "0 mismatch(es)" in run.stdout, run.stdout + run.stderr


def test_grid_map_covers_every_head_and_block_once(tmp_path):
    """The kernels' workgroup-to-(head, block) map (tests/c/grid_map_check.cpp),
    built for the host only from the kernels' own header: a bijection for every head
    group size, head order, block order and a range of head and block counts."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc")
    exe = str(tmp_path / "grid_map_check")
    build = subprocess.run([hipcc, "--cuda-host-only", "-O2", "-std=c++17", "-I",
                            os.path.join(ROOT, "exact_tiled_attention_06_amd", "csrc"),
                            os.path.join(ROOT, "tests", "c", "grid_map_check.cpp"), "-o", exe],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "0 failure(s)" in run.stdout, run.stdout + run.stderr
