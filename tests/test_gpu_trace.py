"""FA_TRACE=1: each launch names its kernel instantiation and grid on stderr
(checked in a child process, where the variable is set before the library
reads it)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import torch
import exact_attention_03_amd as fa
dev = "cuda"
q = torch.randn(1, 16, 300, 128, device=dev).to(torch.bfloat16)
k = torch.randn(1, 2, 300, 128, device=dev).to(torch.bfloat16)
v = torch.randn(1, 2, 300, 128, device=dev).to(torch.bfloat16)
o = torch.empty_like(q)
lse = torch.empty(1, 16, 300, device=dev)
fa.fa_forward(q, k, v, o, lse, True, 0.088)
fa.fa_forward_window(q, k, v, o, lse, True, 50, -1, 0.088)
torch.cuda.synchronize()
print("child done", flush=True)
"""


def test_trace_names_the_kernel_and_grid(gpu_lib):
    env = dict(os.environ, FA_TRACE="1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "child done" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("[fa] ")]
    # 16 query heads over 2 K/V heads: G = 8, 8 heads x 32 rows per
    # workgroup, 10 query tiles of 32 rows, 2 units.
    assert lines[0].startswith("[fa] fa_fwd_kernel<d=128, causal=1, paged=0, window=0, sparse=0> grid=20 block=512")
    assert lines[1].startswith("[fa] fa_fwd_kernel<d=128, causal=1, paged=0, window=1, sparse=0> grid=20 block=512")
    assert len(lines) == 2
