"""Build libfa.so (the gfx950 kernels + C ABI) in-tree with hipcc.

Usage: python -m exact_attention_03_amd._build   (or call build()).
No GPU is needed: hipcc cross-compiles for gfx950.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_prefill.hip", "fa_decode.hip", "fa_backward.hip", "fa_prefill_fp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed FP32 VALU forms are kept out of the generated code; hipcc forms them
# on its own from plain float code otherwise.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# Per-source flags. The prefill kernel relies on no NaN semantics (masked
# scores are -inf, never NaN), so fmaxf on MFMA results needs no quieting.
PER_SOURCE = {"fa_prefill.hip": ["-fno-honor-nans"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source for gfx950 and link libfa.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([HIPCC, "--offload-arch=" + ARCH, *COMMON, *DEVICE_FLAGS, *PER_SOURCE.get(src, []),
                         *extra_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        # One compiler process per source, at most MAX_JOBS (default 4) at once.
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "4"))))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for out in pool.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
