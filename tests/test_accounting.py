"""The FLOP and byte helpers of bench.py against closed forms and against the
sizes the pages print.

Pages (cited by title and section):
  * "Variantes d'attention", "Points cles": the K/V cache of one request on a
    70B model with 64 query heads at 128K context is ~336 GB with one K/V
    head per query head and ~42 GB with 8 K/V heads (GQA, 8x less).
  * "Flash Attention : pourquoi ton GPU utilise 85% de VRAM", "L'attention
    classique en 3 etapes": for 6000 tokens, 32 heads, batch 1, FP16, the
    materialised score matrix is 2.3 GB and O (head dim 128) is 48 "Mo".
The rates bench.py reports divide these helpers' results by measured times,
so a wrong count here would move every reported fraction of peak.
"""
import importlib.util
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_accounting", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


@pytest.mark.parametrize("cfg, flops", [
    (dict(B=4, Hq=16, N=2048, d=128), 68719476736.0),      # 4*4*16*2048^2*128/2
    (dict(B=1, Hq=64, N=8192, d=128), 1099511627776.0),    # 4*64*8192^2*128/2 = 2^40
    (dict(B=1, Hq=32, N=65536, d=128), 35184372088832.0),  # 4*32*65536^2*128/2 = 2^45
])
def test_prefill_flops_follow_the_metric_formula(cfg, flops):
    # 4*B*Hq*Nq*Nk*d, halved for causal; the non-causal count is twice that
    assert bench.prefill_flops(cfg["B"], cfg["Hq"], cfg["N"], cfg["N"], cfg["d"], True) == flops
    assert bench.prefill_flops(cfg["B"], cfg["Hq"], cfg["N"], cfg["N"], cfg["d"], False) == 2 * flops


@pytest.mark.parametrize("cfg, q, kv, lse", [
    (dict(B=4, Hq=16, Hkv=16, N=2048), 4 * 16 * 2048 * 128 * 2, 4 * 16 * 2048 * 128 * 2, 4 * 16 * 2048 * 4),
    (dict(B=1, Hq=64, Hkv=8, N=8192), 64 * 8192 * 128 * 2, 8 * 8192 * 128 * 2, 64 * 8192 * 4),
    (dict(B=1, Hq=32, Hkv=8, N=65536), 32 * 65536 * 128 * 2, 8 * 65536 * 128 * 2, 32 * 65536 * 4),
])
def test_prefill_min_bytes_is_q_k_v_o_lse_once(cfg, q, kv, lse):
    # Q and O (same size), K and V (same size), LSE in fp32
    got = bench.prefill_min_bytes(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["N"], 128)
    assert got == 2 * q + 2 * kv + lse
    # the figures quoted beside the configs: 134.7 MB, 304.1 MB, 1350.6 MB
    assert round(got / 1e5) / 10 in (134.7, 304.1, 1350.6)


def test_kv_cache_of_a_70b_request_at_128k():
    # One 128,000-token sequence, 80 layers, head dim 128, bf16/fp16 K and V.
    # decode_bytes counts one layer's K and V plus q, O, LSE and table entries
    # (a few tens of KB); the cache part dominates.
    layers, L = 80, 128000
    mha = bench.decode_bytes([L], 1, 64, 64, 128) * layers
    gqa = bench.decode_bytes([L], 1, 64, 8, 128) * layers
    assert abs(mha / 336e9 - 1) < 0.01
    assert abs(gqa / 42e9 - 1) < 0.01
    kv_only = L * 64 * 128 * 2 * 2 * layers
    assert 0 < mha - kv_only < 1e-4 * kv_only


def test_materialised_score_and_output_sizes():
    # The naive path's S (and P) for 6000 tokens x 32 heads in FP16, and O at
    # head dim 128: O is the output term of prefill_min_bytes.
    B, H, N, d = 1, 32, 6000, 128
    s_bytes = B * H * N * N * 2
    assert round(s_bytes / 1e8) / 10 == 2.3
    total = bench.prefill_min_bytes(B, H, H, N, N, d)
    o_bytes = (total - 4 * B * H * N) // 4      # Q, K, V and O are equal here
    assert o_bytes == B * H * N * d * 2
    assert o_bytes / 1024 / 1000 == 48.0        # the page's "48 Mo" (thousands of KiB)
    # the three materialised tensors of the page's naive path: S, P and O
    assert abs((2 * s_bytes + o_bytes) / 4.6e9 - 1) < 0.02


def test_decode_bytes_closed_form():
    # two sequences of 1 and 33 tokens, Hq=4, Hkv=2, d=64, 16-token pages
    L = [1, 33]
    kv = (1 + 33) * 2 * 64 * 2 * 2
    q_o = 2 * 4 * 64 * 2 * 2
    lse = 2 * 4 * 4
    table = (1 + 3) * 4
    seq_lens = 2 * 4
    assert bench.decode_bytes(L, 2, 4, 2, 64) == kv + q_o + lse + table + seq_lens


def test_decode_overhead_bytes():
    # Tail slots: 15 and 15 unused slots in the last pages of 1 and 33 tokens.
    # Partials: only sequences with several splits write and re-read them.
    L = [1, 33, 2048, 2049, 5000]
    got = bench.decode_overhead_bytes(L, 5, 8, 2, 64, max_seq_len=8192)
    tail = (15 + 15 + 0 + 15 + 8) * 2 * 64 * 2 * 2
    assert got["tail_slots"] == tail
    assert got["split_tokens"] == 2048          # d = 64 never takes the long split
    n = [1, 1, 1, 2, 3]
    assert got["split_partials"] == sum(x for x in n if x > 1) * 8 * (64 * 4 + 4) * 2
    # d = 128 with a grid of >= 2048 long-split workgroups: 4096-token splits
    big = bench.decode_overhead_bytes([4096, 4097], 2, 64, 8, 128, max_seq_len=32768 * 64)
    assert big["split_tokens"] == 4096
    assert big["split_partials"] == 2 * 64 * (128 * 4 + 4) * 2
    small = bench.decode_overhead_bytes([4096, 4097], 2, 64, 8, 128, max_seq_len=8192)
    assert small["split_tokens"] == 2048
    assert small["split_partials"] == (2 + 3) * 64 * (128 * 4 + 4) * 2


def test_bench_decode_overhead_is_small_against_algorithmic_bytes():
    # the timed decode workload: overhead well under 1% of the algorithmic bytes
    import gen
    D = bench.DECODE
    seq_lens, _, _ = gen.decode_layout(D["seed"], D["B"], D["len_lo"], D["len_hi"], D["page"], D["max_pages"])
    alg = bench.decode_bytes(seq_lens, D["B"], D["Hq"], D["Hkv"], D["d"], D["page"])
    ov = bench.decode_overhead_bytes(seq_lens, D["B"], D["Hq"], D["Hkv"], D["d"], D["max_pages"] * D["page"],
                                     D["page"])
    assert ov["split_tokens"] == 4096
    frac = (ov["tail_slots"] + ov["split_partials"]) / alg
    assert 0 < frac < 0.01
    assert np.asarray(seq_lens).min() >= D["len_lo"]
