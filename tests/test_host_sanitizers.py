"""Host sanitizers (CPU only): the C ABI's argument validation (fa_api.cpp)
and the input generator (gen.c), compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc's runtime, preloaded into a child Python),
run test_abi.py and test_gen.py. Any report aborts the child. The kernels
are compiled as usual and never launched: every ABI test fails validation
before a HIP call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import exact_attention_03_amd as fa
import gen
fa.LIB_PATH = {fa_lib!r}
gen._SO = {gen_lib!r}
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                  {abi!r}, {gen_test!r}])
assert fa._lib is None or fa._lib._name == {fa_lib!r}
assert gen._lib is None or gen._lib._name == {gen_lib!r}
sys.exit(int(rc))
"""


def test_abi_and_generator_under_asan_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("LD_PRELOAD is already set by the environment; not replacing it")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's libasan is not installed")
    sys.path.insert(0, ROOT)
    from exact_attention_03_amd import _build
    import gen
    fa_lib = _build.build_host_sanitized(str(tmp_path))
    gen_lib = gen.build_host_sanitized(str(tmp_path))
    script = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), fa_lib=fa_lib, gen_lib=gen_lib,
                          abi=os.path.join(ROOT, "tests", "test_abi.py"),
                          gen_test=os.path.join(ROOT, "tests", "test_gen.py"))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", script], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, env=env, timeout=600)
    print(r.stdout[-3000:])
    assert "AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
    assert r.returncode == 0, r.stdout[-3000:]
    assert " passed" in r.stdout
