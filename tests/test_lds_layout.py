"""The LDS tile layout the kernels rely on, checked on the host.

The staged-tile helpers in exact_attention_03_amd/csrc/fa_lds.h are pure
integer functions (also callable from host code). tests/lds_layout_check.hip
calls those very functions and checks, exhaustively: the chunk swizzle is a
bijection that depends on the row modulo 16; the K-fragment offsets of every
k-step and the transposing-read offsets of every dim block differ from the
block-0 offset by an xor with a constant (the kernels keep only the base);
one lane offset serves every copy block of a wave when tiles start at rows
that are multiples of 16 (the scalar-base copies); the permuted K-row order
is a bijection. Compiled with hipcc for the host; no GPU needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_lds_layout_properties(tmp_path):
    exe = tmp_path / "lds_layout_check"
    src = os.path.join(ROOT, "tests", "lds_layout_check.hip")
    inc = os.path.join(ROOT, "exact_attention_03_amd", "csrc")
    build = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", inc, "-x", "hip", src,
                            "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-3000:]
    assert "all properties hold" in run.stdout


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_fast_divisor_matches_integer_division(tmp_path):
    """fast_div() (csrc/fa_divide.h), which the kernels use to map workgroup
    and step indices, equals n / d: exhaustively for small pairs, at every
    quotient boundary for divisors up to 2^17, and on random pairs."""
    exe = tmp_path / "fastdiv_check"
    src = os.path.join(ROOT, "tests", "fastdiv_check.hip")
    inc = os.path.join(ROOT, "exact_attention_03_amd", "csrc")
    build = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", inc, "-x", "hip", src,
                            "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-3000:]
    assert "all properties hold" in run.stdout
