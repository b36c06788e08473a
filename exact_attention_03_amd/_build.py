"""Build libfa.so (the gfx950 kernels + C ABI) in-tree with hipcc.

Usage: python -m exact_attention_03_amd._build   (or call build()).
No GPU is needed: hipcc cross-compiles for gfx950.

build_host_sanitized() makes a second copy of the library whose host code
(the C ABI's argument validation, fa_api.cpp) is compiled by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer; the kernels are compiled
as usual. tests/test_host_sanitizers.py loads it (with gcc's libasan
preloaded) under the ABI and generator tests.
"""
from __future__ import annotations

import hashlib
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


def _compile_all(tmp, sources, extra_flags=()):
    objs, cmds = [], []
    for src in sources:
        obj = os.path.join(tmp, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, "--offload-arch=" + ARCH, *COMMON, *DEVICE_FLAGS, *PER_SOURCE.get(src, []),
                     *extra_flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # One compiler process per source, at most MAX_JOBS (default 4) at once.
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "4"))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        outs = list(pool.map(_run, cmds))
    return objs, outs


# Host sanitizers for the ABI layer: gcc's runtime (g++ compiles fa_api.cpp,
# which holds no device code, against the HIP headers).
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str) -> str:
    """libfa_hostsan.so in out_dir: fa_api.cpp under ASan + UBSan (g++), the
    kernels as in build()."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libfa_hostsan.so")
    with tempfile.TemporaryDirectory(prefix="fa_build_san_") as tmp:
        objs, _ = _compile_all(tmp, [s for s in SOURCES if s.endswith(".hip")])
        api = os.path.join(tmp, "fa_api_san.o")
        _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SANITIZE, "-c", os.path.join(CSRC, "fa_api.cpp"),
              "-o", api])
        _run(["g++", "-shared", *SANITIZE, api, *objs, "-L", "/opt/rocm/lib", "-lamdhip64",
              "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    return lib


STAMP = LIB + ".srchash"


def source_digest(extra_flags=()) -> str:
    """sha256 of every kernel / ABI source, the public header and the flags:
    written next to libfa.so by build(), compared by load() so that a library
    older than its sources is never used."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))
    for name in files:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "fa.h"), "rb") as fh:
        h.update(fh.read())
    h.update(repr((COMMON[:5], DEVICE_FLAGS, sorted(PER_SOURCE.items()), list(extra_flags))).encode())
    return h.hexdigest()


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source for gfx950 and link libfa.so next to this file."""
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs, outs = _compile_all(tmp, SOURCES, extra_flags)
        for out in outs:
            if verbose and out.strip():
                print(out)
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    with open(STAMP, "w") as fh:
        fh.write(source_digest(extra_flags) + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
