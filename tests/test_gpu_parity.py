"""GPU parity: the HIP kernels through the C ABI against the fp64 CPU oracle on
the same seeded bf16 inputs, element by element (small and ragged shapes, the
five workload configurations) to the acceptance bar in fa_cases."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
from fa_cases import (BackwardCase, bf16_mean_bar, DecodeCase, PagedPrefillCase, PrefillCase, bf16_dev_to_f64, compare,
                      compare_grads, f64_to_bf16_bits, fp8_bars, fp8_bound_terms, say, to_dev_bf16)

pytestmark = pytest.mark.gpu


def check_prefill(case: PrefillCase, rows=None, what="", bf16_bound=False):
    say("prefill %s B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d seed=%d" % (
        what, case.B, case.Hq, case.Hkv, case.Nq, case.Nk, case.d, case.causal, case.seed))
    o, lse = case.run_gpu()
    o64 = bf16_dev_to_f64(o)
    l32 = lse.cpu().numpy().astype(np.float64)
    o_ref, l_ref = case.oracle(rows=rows)
    if rows is not None:
        r = np.asarray(rows)
        if r.ndim == 1:
            o64, l32 = o64[:, :, r], l32[:, :, r]
        else:
            bi = np.arange(case.B)[:, None, None]
            hi = np.arange(case.Hq)[None, :, None]
            o64, l32 = o64[bi, hi, r], l32[bi, hi, r]
    vmax = float(np.abs(oracle.bf16_bits_to_f64(case.v_bits)).max()) if bf16_bound else None
    mbar = bf16_mean_bar(case, rows=rows) if bf16_bound else None
    return compare(o64, l32, o_ref, l_ref, what, v_absmax=vmax, mean_bar=mbar)


SMALL = [  # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 32, 64, 128, False),
    (2, 8, 2, 300, 300, 128, True),     # several tiles, ragged tail, G=4
    (1, 8, 2, 77, 333, 128, True),      # Nq < Nk: bottom-right causal diagonal
    (2, 4, 2, 200, 129, 64, False),     # d=64, ragged Nk
    (1, 16, 1, 100, 100, 128, True),    # MQA, G=16 (two head subsets of 8)
    (1, 6, 2, 150, 150, 64, True),      # G=3 (one head per block group)
    (3, 2, 2, 257, 257, 128, True),     # MHA, G=1, three q tiles per head
    (1, 64, 8, 96, 96, 128, True),      # G=8 packing
    (1, 4, 4, 1, 1, 128, True),         # single token
    (1, 2, 1, 5, 700, 64, False),       # tiny Nq, long Nk
    (1, 4, 2, 600, 600, 128, True),     # G=2: 2 heads x 4 query blocks per workgroup
    (1, 8, 8, 256, 257, 128, True),     # Nk = 2 tiles + 1 key: one-key last tile, shifted diagonal
    (1, 16, 2, 1000, 1000, 64, True),   # d=64, G=8, many tiles, ragged tail
    (2, 2, 2, 130, 1000, 128, False),   # G=1 non-causal, Nk not a tile multiple
    (1, 2, 1, 300, 100, 128, True),     # Nq > Nk: some waves of a workgroup have no visible keys
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(shape, gpu_lib):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    check_prefill(PrefillCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=7 + Nq), what="small")


def test_rows_without_visible_keys(gpu_lib):
    # causal with Nq > Nk: the first Nq - Nk rows see no key -> O = 0, LSE = -inf
    check_prefill(PrefillCase(1, 4, 2, 100, 40, 128, True, seed=3), what="Nq>Nk")


def test_no_keys(gpu_lib):
    check_prefill(PrefillCase(1, 2, 1, 50, 0, 64, False, seed=4), what="Nk=0")


def test_large_logits_sigma(gpu_lib):
    # wide score range (sigma 3): exercises the lazy rescale path repeatedly
    check_prefill(PrefillCase(1, 8, 2, 520, 520, 128, True, seed=5, sigma=3.0), what="sigma3", bf16_bound=True)


def test_config1_tiny_noncausal(gpu_lib):
    check_prefill(PrefillCase(1, 1, 1, 128, 128, 64, False, seed=1001, scale=0.125), what="c1")


def test_config2_causal_mha(gpu_lib):
    check_prefill(PrefillCase(4, 16, 16, 2048, 2048, 128, True, seed=1002), what="c2")


def test_config3_causal_gqa_sampled_rows_and_one_head_group(gpu_lib):
    """The whole c3 launch on the GPU: 64 sampled rows of every query head,
    and every row of K/V head 5's group (query heads 40..47; a head group's
    output depends on that group's inputs alone, so the oracle runs on its
    slice)."""
    case = PrefillCase(1, 64, 8, 8192, 8192, 128, True, seed=1003)
    say("prefill c3 B=1 Hq=64 Hkv=8 N=8192 d=128 causal seed=1003")
    o, lse = case.run_gpu()
    o64 = bf16_dev_to_f64(o)
    l64 = lse.cpu().numpy().astype(np.float64)
    rows = np.stack([np.stack([gen.row_sample(1003, 8192, 64, salt=h) for h in range(64)])])
    o_ref, l_ref = case.oracle(rows=rows)
    bi, hi = np.arange(1)[:, None, None], np.arange(64)[None, :, None]
    compare(o64[bi, hi, rows], l64[bi, hi, rows], o_ref, l_ref, "c3 (64 rows/head)")
    g = 5
    f = oracle.bf16_bits_to_f64
    o_ref, l_ref = oracle.attention_naive(f(case.q_bits[:, 8 * g:8 * g + 8]), f(case.k_bits[:, g:g + 1]),
                                          f(case.v_bits[:, g:g + 1]), case.scale, True)
    compare(o64[:, 8 * g:8 * g + 8], l64[:, 8 * g:8 * g + 8], o_ref, l_ref, "c3 (K/V head 5, all rows)")


def test_config4_long_context_sampled_rows(gpu_lib):
    case = PrefillCase(1, 32, 8, 65536, 65536, 128, True, seed=1004, sigma=0.5)
    rows = np.stack([np.stack([gen.row_sample(1004, 65536, 256, salt=h) for h in range(32)])])
    check_prefill(case, rows=rows, what="c4 (256 rows/head)")


# ---------------------------------------------------------------- decode

def check_decode(case: DecodeCase, what=""):
    say("decode %s B=%d Hq=%d Hkv=%d d=%d lens=[%s] seed=%d" % (
        what, case.B, case.Hq, case.Hkv, case.d,
        ",".join(map(str, case.seq_lens[:8])) + ("..." if case.B > 8 else ""), case.seed))
    o, lse = case.run_gpu()
    o_ref, l_ref = case.oracle()
    return compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, what)


@pytest.mark.parametrize("lens,Hq,Hkv,d", [
    ([1, 16, 17, 1000, 2500], 8, 1, 128),
    ([1023, 1024, 1025, 2048, 3333], 64, 8, 128),
    ([5, 700, 4100], 16, 4, 64),
    ([300, 9000], 32, 2, 128),          # G=16
    ([2000, 50], 4, 4, 128),            # MHA decode
])
def test_decode_small(lens, Hq, Hkv, d, gpu_lib):
    check_decode(DecodeCase(len(lens), Hq, Hkv, d, seed=11 + len(lens), seq_lens=lens), what="small")


def test_decode_long_split_boundaries(gpu_lib):
    # d = 128 with B * Hkv * ceil(max_seq_len / 4096) >= 2048 workgroups runs
    # 4096-token splits: 32 sequences, Hkv = 8, max_seq_len 32768. Lengths sit
    # on and around the split and page edges (one split, a 1-token second
    # split, several splits with ragged tails, an empty sequence).
    edges = [0, 1, 16, 2047, 2048, 2049, 4095, 4096, 4097, 6000, 8191, 8192, 8193, 12289, 16400, 32768]
    rest = [int(x) for x in np.random.default_rng(13).integers(1, 32769, 32 - len(edges))]
    lens = edges + rest
    assert 32 * 8 * (32768 // 4096) >= 2048
    check_decode(DecodeCase(32, 32, 8, 128, seed=13, seq_lens=lens, max_seq_len=32768), what="long split")


def test_decode_empty_sequence(gpu_lib):
    check_decode(DecodeCase(3, 8, 1, 128, seed=12, seq_lens=[0, 33, 0]), what="L=0")


def test_config5_paged_decode(gpu_lib):
    check_decode(DecodeCase(64, 64, 8, 128, seed=1005, len_lo=512, len_hi=32768,
                            max_pages_per_seq=2048, max_seq_len=32768), what="c5")



# ---- paged (chunked) prefill ----

def check_paged_prefill(case: PagedPrefillCase, what=""):
    say("paged prefill %s B=%d Hq=%d Hkv=%d d=%d causal=%d lens=%s chunks=%s seed=%d" % (
        what, case.B, case.Hq, case.Hkv, case.d, case.causal, list(case.seq_lens)[:8], list(case.q_lens)[:8],
        case.seed))
    o, lse = case.run_gpu()
    o_ref, l_ref = case.oracle()
    return compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, what)


PAGED_PREFILL = [  # Hq, Hkv, d, causal, seq_lens, q_lens
    (8, 1, 128, True, [300, 17, 1000, 64], [300, 5, 129, 1]),   # full chunk, short, ragged, decode-like
    (16, 2, 128, True, [513, 40], [200, 40]),                   # G=8 packing, chunk == cache
    (4, 4, 64, True, [77, 256, 1], [30, 256, 1]),               # MHA, d=64
    (6, 2, 128, False, [100, 333], [64, 7]),                    # non-causal, G=3
    (8, 2, 128, True, [0, 50, 20], [4, 0, 30]),                 # empty cache; empty chunk; chunk > cache
]


@pytest.mark.parametrize("Hq,Hkv,d,causal,lens,chunks", PAGED_PREFILL,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, list) else str(v))
def test_paged_prefill(Hq, Hkv, d, causal, lens, chunks, gpu_lib):
    check_paged_prefill(PagedPrefillCase(Hq, Hkv, d, seed=31 + len(lens), seq_lens=lens, q_lens=chunks,
                                         causal=causal), what="small")


def test_paged_prefill_chunked_long_context(gpu_lib):
    # 8 sequences, caches of 1..8K tokens, 512-token chunks: a chunked-prefill
    # step of a 64/8-head model.
    r = np.random.default_rng(41)
    lens = [int(x) for x in r.integers(512, 8192, 8)]
    check_paged_prefill(PagedPrefillCase(64, 8, 128, seed=41, seq_lens=lens, q_lens=[512] * 8), what="long")




def test_paged_prefill_timed_workload(gpu_lib):
    # The timed chunked prefill: 8 sequences with 2K-16K cached tokens (seed
    # 1006, table of 1024 pages per sequence), a 1024-token causal chunk each,
    # GQA 64/8, d=128; the whole batch on the GPU. Heads are independent, so
    # the oracle checks K/V head group 3 of the shortest and longest sequence.
    import exact_attention_03_amd as fa
    B, Hq, Hkv, d, chunk, seed = 8, 64, 8, 128, 1024, 1006
    lens, table, total = gen.decode_layout(seed, B, 2048, 16384, 16, 1024)
    cu = (np.arange(B + 1) * chunk).astype(np.int32)
    q_bits = gen.normal_bf16(seed, gen.STREAM_Q, (B * chunk, Hq, d))
    k_bits = gen.normal_bf16(seed, gen.STREAM_K, (total, Hkv, 16, d))
    v_bits = gen.normal_bf16(seed, gen.STREAM_V, (total, Hkv, 16, d))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    say("paged prefill timed workload: lens=%s pages=%d" % (list(lens), total))
    o = torch.full((B * chunk, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B * chunk, Hq), float("nan"), dtype=torch.float32, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    fa.fa_paged_prefill(to_dev_bf16(q_bits), to_dev_bf16(k_bits), to_dev_bf16(v_bits), dev(table), dev(lens),
                        dev(cu), o, lse, chunk, True, scale)
    torch.cuda.synchronize()
    og, lg = bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64)
    g = 3
    hs = slice(8 * g, 8 * g + 8)
    for b in (int(np.argmin(lens)), int(np.argmax(lens))):
        r = slice(int(cu[b]), int(cu[b + 1]))
        o_ref, l_ref = oracle.paged_prefill(q_bits[r][:, hs], k_bits[:, g:g + 1], v_bits[:, g:g + 1], table[b:b + 1],
                                            lens[b:b + 1], np.array([0, chunk]), scale, True)
        compare(og[r][:, hs], lg[r][:, hs], o_ref, l_ref, "timed paged prefill, sequence %d (L=%d)" % (b, lens[b]))


PAGED_PREFILL_WINDOWS = [  # Hq, Hkv, d, causal, (left, right), seq_lens, q_lens
    (8, 1, 128, True, (255, -1), [2000, 300, 17], [300, 300, 5]),      # pages below the band skipped
    (8, 2, 128, True, (0, -1), [129, 40], [129, 3]),                   # each row sees itself only
    (6, 2, 128, False, (100, 50), [1000, 333], [260, 7]),              # two-sided, right bound past the end
    (4, 4, 64, False, (-1, 20), [77, 256, 1], [30, 256, 1]),           # right bound only, d=64 MHA
    (8, 2, 64, True, (31, -1), [0, 50, 20, 700], [4, 0, 30, 129]),     # empty cache / chunk, chunk > cache
    (16, 2, 128, True, (1000, -1), [3000, 1100], [1, 200]),            # decode-like row, G=8 packing
]


@pytest.mark.parametrize("Hq,Hkv,d,causal,window,lens,chunks", PAGED_PREFILL_WINDOWS,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, (list, tuple)) else str(v))
def test_paged_prefill_window(Hq, Hkv, d, causal, window, lens, chunks, gpu_lib):
    check_paged_prefill(PagedPrefillCase(Hq, Hkv, d, seed=61 + len(lens), seq_lens=lens, q_lens=chunks,
                                         causal=causal, window=window), what="window %s" % (window,))


def test_paged_prefill_window_long_context(gpu_lib):
    # Chunked prefill of a 64/8-head model with a 1024-token causal window:
    # 8 caches of 1..8K tokens, 512-token chunks.
    r = np.random.default_rng(42)
    lens = [int(x) for x in r.integers(512, 8192, 8)]
    check_paged_prefill(PagedPrefillCase(64, 8, 128, seed=42, seq_lens=lens, q_lens=[512] * 8,
                                         window=(1023, -1)), what="long window")

# ---- sliding window ----

WINDOWS = [  # B, Hq, Hkv, Nq, Nk, d, causal, (left, right)
    (1, 8, 1, 1000, 1000, 128, True, (256, -1)),    # causal sliding window, tiles skipped below
    (1, 64, 8, 600, 600, 128, True, (17, -1)),      # window narrower than a tile, G=8 packing
    (1, 4, 4, 700, 700, 128, False, (64, 64)),      # symmetric local window, non-causal, MHA
    (2, 4, 2, 100, 900, 128, True, (200, -1)),      # Nq < Nk: bottom-right positions
    (1, 2, 1, 300, 300, 64, True, (0, -1)),         # each query sees only its own key; d=64
    (1, 6, 2, 257, 513, 64, False, (-1, 3)),        # right bound only (non-causal), G=3
    (1, 8, 2, 400, 400, 128, True, (1000, -1)),     # window wider than the sequence: plain causal
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,win", WINDOWS,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_sliding_window(B, Hq, Hkv, Nq, Nk, d, causal, win, gpu_lib):
    check_prefill(PrefillCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=61 + Nq, window=win), what="window %s" % (win,))


def test_sliding_window_long_sampled_rows(gpu_lib):
    # 8K causal GQA with a 4096-key window: sampled rows against the oracle.
    case = PrefillCase(1, 64, 8, 8192, 8192, 128, True, seed=1007, window=(4096, -1))
    rows = gen.row_sample(1007, 8192, 64)
    check_prefill(case, rows=rows, what="window 4096 8K")


# Grids of more workgroups than the MI355X has CUs (several rounds per CU):
# ragged lengths, both head dims, GQA packings of 8, 3 and 1 heads per
# workgroup, Nq < Nk, Nq > Nk (rows with no key), one-tile workgroups.
MANY = [  # B, Hq, Hkv, Nq, Nk, d, causal   (workgroups: > 256)
    (4, 32, 4, 777, 777, 128, True),      # G=8: 32-row tiles, ragged (400)
    (4, 32, 4, 777, 777, 128, False),     # (400)
    (8, 32, 32, 300, 300, 128, True),     # G=1: 256-row tiles (512)
    (4, 16, 2, 1030, 1030, 64, True),     # d=64 (264)
    (20, 16, 2, 200, 1500, 128, True),    # Nq < Nk (280)
    (4, 16, 2, 1400, 300, 128, True),     # Nq > Nk: leading rows see no key (352)
    (5, 24, 8, 513, 513, 128, True),      # G=3: 3 head subsets per K/V head (360)
    (40, 8, 8, 97, 97, 128, False),       # one key tile each (320)
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", MANY,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_prefill_many_workgroups(B, Hq, Hkv, Nq, Nk, d, causal, gpu_lib):
    check_prefill(PrefillCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=91 + Nq), what="many workgroups")


SPARSE = [  # B, Hq, Hkv, Nq, Nk, d, causal, percent, mask batch dim, mask head dim
    (1, 8, 1, 1000, 1000, 128, True, 50, 1, 8),     # G=8: 8 heads per workgroup, each its own mask
    (1, 2, 2, 700, 900, 128, False, 40, 1, 2),      # G=1: two query blocks per workgroup
    (2, 8, 2, 513, 513, 64, True, 60, 2, 8),        # per batch and head, d=64, ragged
    (1, 4, 4, 300, 1200, 128, True, 30, 1, 1),      # one mask for all, Nq < Nk
    (1, 4, 2, 1030, 260, 128, False, 70, 1, 4),     # Nq > Nk, G=2
    (1, 2, 1, 640, 640, 128, True, 10, 1, 2),       # very sparse: empty rows of blocks
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,pct,mb,mh", SPARSE,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_block_sparse(B, Hq, Hkv, Nq, Nk, d, causal, pct, mb, mh, gpu_lib):
    mask = gen.random_block_mask(71 + Nq, (mb, mh, -(-Nq // 128), -(-Nk // 128)), pct)
    check_prefill(PrefillCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=71 + Nq, block_mask=mask),
                  what="block-sparse %d%%" % pct)


def test_block_sparse_all_ones_matches_dense_bitwise(gpu_lib):
    # With every block set the sparse kernel visits the same tiles in the same
    # order with the same masks as the dense one: identical bits.
    for (B, Hq, Hkv, N, d, causal) in ((1, 8, 2, 777, 128, True), (1, 2, 2, 500, 64, False)):
        dense = PrefillCase(B, Hq, Hkv, N, N, d, causal, seed=81)
        sparse = PrefillCase(B, Hq, Hkv, N, N, d, causal, seed=81,
                             block_mask=np.ones((1, 1, -(-N // 128), -(-N // 128)), np.uint8))
        o1, l1 = dense.run_gpu()
        o2, l2 = sparse.run_gpu()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_block_sparse_all_zero_is_empty(gpu_lib):
    case = PrefillCase(1, 4, 1, 300, 300, 128, True, seed=82, block_mask=np.zeros((1, 1, 3, 3), np.uint8))
    o, lse = case.run_gpu()
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


def test_block_sparse_local_global_long_sampled_rows(gpu_lib):
    # 8K causal GQA, local (16 blocks) + global (first block) pattern.
    mask = gen.local_global_block_mask(64, 64, 16, 1)[None, None]
    case = PrefillCase(1, 64, 8, 8192, 8192, 128, True, seed=1008, block_mask=mask)
    rows = gen.row_sample(1008, 8192, 64)
    check_prefill(case, rows=rows, what="local+global 8K")


BACKWARD = [  # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 64, 64, 128, False),
    (1, 2, 1, 128, 128, 128, True),
    (1, 4, 2, 100, 130, 128, True),      # ragged, Nq < Nk
    (2, 8, 2, 257, 257, 128, True),      # GQA 4, ragged tail, two batches
    (1, 4, 4, 60, 300, 128, True),       # Nq << Nk
    (1, 4, 2, 300, 100, 128, True),      # Nq > Nk: leading rows see no key
    (1, 8, 1, 200, 333, 64, False),      # d=64, MQA
    (1, 6, 2, 129, 129, 64, True),       # d=64, G=3
    (1, 16, 2, 1024, 1024, 128, True),   # many tiles
    (1, 8, 8, 200, 700, 128, False),     # non-causal, 11 key tiles of 64, the last one ragged
    (1, 16, 2, 333, 333, 64, True),      # d=64, G=8, ragged
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", BACKWARD,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_backward(B, Hq, Hkv, Nq, Nk, d, causal, gpu_lib):
    case = BackwardCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=101 + Nq)
    say("backward B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d" % (B, Hq, Hkv, Nq, Nk, d, causal))
    o, lse, dq, dk, dv = case.oracle()
    got = case.run_gpu(o, lse)
    compare_grads(got, (dq, dk, dv), "backward")


BACKWARD_WINDOWS = [  # B, Hq, Hkv, Nq, Nk, d, causal, (left, right)
    (1, 4, 2, 500, 500, 128, True, (100, -1)),     # causal sliding window, key tiles skipped below
    (1, 8, 2, 300, 300, 128, True, (17, -1)),      # window narrower than a tile
    (1, 4, 4, 400, 400, 128, False, (64, 64)),     # symmetric local window, non-causal, MHA
    (2, 4, 2, 100, 700, 128, True, (200, -1)),     # Nq < Nk: bottom-right positions
    (1, 6, 2, 257, 513, 64, False, (-1, 3)),       # right bound only, d=64, G=3
    (1, 2, 1, 300, 300, 64, True, (0, -1)),        # each query sees only its own key
    (1, 8, 2, 400, 400, 128, True, (1000, -1)),    # window wider than the sequence: plain causal
    (1, 4, 2, 300, 100, 128, True, (30, -1)),      # Nq > Nk: leading rows see no key
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,win", BACKWARD_WINDOWS,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_backward_window(B, Hq, Hkv, Nq, Nk, d, causal, win, gpu_lib):
    case = BackwardCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=121 + Nq, window=win)
    say("backward window %s B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d" % (win, B, Hq, Hkv, Nq, Nk, d, causal))
    o, lse, dq, dk, dv = case.oracle()
    compare_grads(case.run_gpu(o, lse), (dq, dk, dv), "backward window")


def test_backward_window_after_gpu_forward(gpu_lib):
    case = BackwardCase(1, 8, 2, 600, 600, 128, True, seed=131, window=(150, -1))
    _, _, dq, dk, dv = case.oracle()
    compare_grads(case.run_gpu(), (dq, dk, dv), "window forward+backward")


def test_backward_config3_head_group(gpu_lib):
    # The timed backward: causal GQA 64/8 N=8192 d=128 (the prefill inputs,
    # dO from its own stream), fed by the GPU forward's O and LSE, the whole
    # problem on the GPU. A K/V head's gradients, and those of its 8 query
    # heads, depend on that head group alone, so the oracle checks group 5 in
    # full (every row of dQ, dK and dV).
    case = BackwardCase(1, 64, 8, 8192, 8192, 128, True, seed=1003)
    say("backward c3 B=1 Hq=64 Hkv=8 N=8192 d=128 causal, oracle on K/V head 5")
    dq_g, dk_g, dv_g = case.run_gpu()
    g, f = 5, oracle.bf16_bits_to_f64
    hs = slice(8 * g, 8 * g + 8)
    ref = oracle.attention_backward(f(case.q_bits[:, hs]), f(case.k_bits[:, g:g + 1]), f(case.v_bits[:, g:g + 1]),
                                    f(case.do_bits[:, hs]), case.scale, True)
    compare_grads((dq_g[:, hs], dk_g[:, g:g + 1], dv_g[:, g:g + 1]), ref, "c3 backward")


def test_backward_after_gpu_forward(gpu_lib):
    # The training-step pipeline: fa_forward's own O and LSE feed fa_backward.
    case = BackwardCase(1, 8, 2, 500, 500, 128, True, seed=111)
    _, _, dq, dk, dv = case.oracle()
    compare_grads(case.run_gpu(), (dq, dk, dv), "forward+backward")



BACKWARD_SPARSE = [  # B, Hq, Hkv, Nq, Nk, d, causal, percent, mask batch dim, mask head dim
    (1, 8, 1, 1000, 1000, 128, True, 50, 1, 8),      # G=8: 8 heads per dq workgroup, each its own mask
    (1, 2, 2, 700, 900, 128, False, 40, 1, 2),       # G=1: two query blocks per dq workgroup
    (2, 8, 2, 513, 513, 64, True, 60, 2, 8),         # per batch and head, d=64, ragged
    (1, 4, 4, 300, 1200, 128, True, 30, 1, 1),       # one mask for all, Nq < Nk
    (1, 4, 2, 1030, 260, 128, False, 70, 1, 4),      # Nq > Nk, G=2
    (1, 2, 1, 640, 640, 128, True, 10, 1, 2),        # very sparse: key blocks no query sees
    (1, 16, 1, 4160, 300, 128, False, 50, 1, 16),    # ~520 visible dK/dV steps per key block: cut into runs, combined
    (1, 16, 16, 38400, 300, 64, False, 40, 1, 16),   # G=1, 600 steps per key block, B * Hkv = 16: one run
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,pct,mb,mh", BACKWARD_SPARSE,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_backward_block_sparse(B, Hq, Hkv, Nq, Nk, d, causal, pct, mb, mh, gpu_lib):
    mask = gen.random_block_mask(141 + Nq, (mb, mh, -(-Nq // 128), -(-Nk // 128)), pct)
    case = BackwardCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=141 + Nq, block_mask=mask)
    say("backward block-sparse %d%% B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d mask %s"
        % (pct, B, Hq, Hkv, Nq, Nk, d, causal, mask.shape))
    o, lse, dq, dk, dv = case.oracle()
    compare_grads(case.run_gpu(o, lse), (dq, dk, dv), "backward block-sparse")


@pytest.mark.parametrize("Hq,Nq,Nk", [(4, 500, 500), (8, 4480, 300)], ids=["one_run", "two_runs"])
def test_backward_block_sparse_cleared_blocks_get_zero_gradients(Hq, Nq, Nk, gpu_lib):
    # Key block 1 is seen by no query and query block 2 sees nothing: their
    # dK, dV and dQ rows are exactly zero, the rest matches the oracle. In the
    # second shape key blocks 0 and 2 have 8 x 68 visible dK/dV steps, cut
    # into runs and combined; key block 1 has none.
    mask = np.ones((1, 1, -(-Nq // 128), -(-Nk // 128)), np.uint8)
    mask[..., 1] = 0
    mask[..., 2, :] = 0
    case = BackwardCase(1, Hq, 1, Nq, Nk, 128, False, seed=151, block_mask=mask)
    o, lse, dq, dk, dv = case.oracle()
    got = case.run_gpu(o, lse)
    compare_grads(got, (dq, dk, dv), "cleared blocks")
    assert (got[1][:, :, 128:256] == 0).all() and (got[2][:, :, 128:256] == 0).all()
    assert (got[0][:, :, 256:384] == 0).all()


def test_backward_block_sparse_all_ones_matches_dense(gpu_lib):
    # Every block set: the sparse kernels visit the same tiles and steps in
    # the same order as fa_backward (each dK/dV walk spans its key block's
    # query tiles up to the last one, so it starts at the top as dense does),
    # and where each key block's dK/dV walk is one run the gradients agree bit
    # for bit. Where a walk is cut into runs (the last shape: up to 16 x 65
    # steps per key block) the runs' fp32 partials are summed in run order,
    # which rounds differently from one long sum: dQ still agrees bit for
    # bit, dK and dV to the gradient bar.
    for (B, Hq, Hkv, N, d, causal) in [(1, 8, 2, 1000, 128, True), (2, 6, 3, 333, 64, False),
                                       (1, 16, 16, 38400, 64, True), (1, 16, 1, 4160, 128, True)]:
        ones = np.ones((1, 1, -(-N // 128), -(-N // 128)), np.uint8)
        dense = BackwardCase(B, Hq, Hkv, N, N, d, causal, seed=161 + N)
        sparse = BackwardCase(B, Hq, Hkv, N, N, d, causal, seed=161 + N, block_mask=ones)
        say("backward all-ones mask vs dense B=%d Hq=%d Hkv=%d N=%d d=%d causal=%d" % (B, Hq, Hkv, N, d, causal))
        got_d, got_s = dense.run_gpu(), sparse.run_gpu()
        if Hkv == 1 and N == 4160:
            assert np.array_equal(got_d[0], got_s[0]), "dQ"
            compare_grads(got_s, got_d, "all-ones, runs combined")
        else:
            for a, b, name in zip(got_d, got_s, ("dQ", "dK", "dV")):
                assert np.array_equal(a, b), name


def test_backward_block_sparse_local_global_head_group(gpu_lib):
    # The block-sparse prefill's pattern at 8K (causal GQA 64/8, d=128, local
    # 16 blocks + the first block), forward and backward on the GPU; the
    # oracle checks K/V head 2 and its 8 query heads in full.
    mask = gen.local_global_block_mask(64, 64, 16, 1)[None, None]
    case = BackwardCase(1, 64, 8, 8192, 8192, 128, True, seed=1008, block_mask=mask)
    say("backward block-sparse local+global 8K, oracle on K/V head 2")
    dq_g, dk_g, dv_g = case.run_gpu()
    g, f = 2, oracle.bf16_bits_to_f64
    hs = slice(8 * g, 8 * g + 8)
    ref = oracle.attention_backward(f(case.q_bits[:, hs]), f(case.k_bits[:, g:g + 1]), f(case.v_bits[:, g:g + 1]),
                                    f(case.do_bits[:, hs]), case.scale, True, block_mask=mask)
    compare_grads((dq_g[:, hs], dk_g[:, g:g + 1], dv_g[:, g:g + 1]), ref, "local+global 8K backward")


# ---- FP8 ----

def _fp8_inputs(seed, B, Hq, Hkv, Nq, Nk, d, sigma=1.0):
    q = oracle.bf16_bits_to_f64(gen.normal_bf16(seed, gen.STREAM_Q, (B, Hq, Nq, d), sigma))
    k = oracle.bf16_bits_to_f64(gen.normal_bf16(seed, gen.STREAM_K, (B, Hkv, Nk, d), sigma))
    v = oracle.bf16_bits_to_f64(gen.normal_bf16(seed, gen.STREAM_V, (B, Hkv, Nk, d), sigma))
    return q, k, v


@pytest.mark.parametrize("shape", [(1, 2, 300, 128, 128), (2, 3, 129, 64, 128), (1, 1, 1000, 128, 1000),
                                   (1, 2, 64, 128, 7)], ids=str)
def test_quantize_fp8_bit_exact(shape, gpu_lib):
    import exact_attention_03_amd as fa
    B, H, N, d, block = shape
    bits = gen.normal_bf16(131 + N, gen.STREAM_Q, (B, H, N, d), 2.0)
    bits[0, 0, :min(N, block)] = 0                      # an all-zero block
    x = oracle.bf16_bits_to_f64(bits)
    ref_codes, ref_scales = oracle.quantize_fp8(x, block)
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, -(-N // block)), dtype=torch.float32, device="cuda")
    fa.fa_quantize_fp8(to_dev_bf16(bits), codes, scales, block)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_scales)
    got = codes.cpu().numpy()
    assert np.array_equal(got, ref_codes), "codes differ at %d places" % int((got != ref_codes).sum())


FP8 = [  # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 2, 1, 128, 128, 128, False),
    (1, 4, 2, 300, 300, 128, True),
    (2, 8, 2, 257, 513, 128, True),      # Nq < Nk, ragged
    (1, 4, 4, 400, 100, 128, True),      # Nq > Nk: rows without keys
    (1, 8, 1, 200, 333, 64, False),
    (1, 6, 2, 1000, 1000, 64, True),
    (1, 16, 2, 2048, 2048, 128, True),
]


def check_fp8(B, Hq, Hkv, Nq, Nk, d, causal, seed, gpu_quantize=False, inputs=None, rows=None):
    import exact_attention_03_amd as fa
    say("fp8 B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d seed=%d gpu_quantize=%d" % (
        B, Hq, Hkv, Nq, Nk, d, causal, seed, gpu_quantize))
    q, k, v = _fp8_inputs(seed, B, Hq, Hkv, Nq, Nk, d) if inputs is None else inputs
    qc, qs = oracle.quantize_fp8(q, 128)
    kc, ks = oracle.quantize_fp8(k, 128)
    vc, vs = oracle.quantize_fp8(v, max(1, Nk))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if gpu_quantize:  # the library's own quantizer feeds the kernel
        cq, sq_ = torch.empty(q.shape, dtype=torch.uint8, device="cuda"), torch.empty(qs.shape, device="cuda")
        ck, sk_ = torch.empty(k.shape, dtype=torch.uint8, device="cuda"), torch.empty(ks.shape, device="cuda")
        cv, sv_ = torch.empty(v.shape, dtype=torch.uint8, device="cuda"), torch.empty(vs.shape, device="cuda")
        from fa_cases import f64_to_bf16_bits
        fa.fa_quantize_fp8(to_dev_bf16(f64_to_bf16_bits(q)), cq, sq_, 128)
        fa.fa_quantize_fp8(to_dev_bf16(f64_to_bf16_bits(k)), ck, sk_, 128)
        fa.fa_quantize_fp8(to_dev_bf16(f64_to_bf16_bits(v)), cv, sv_, max(1, Nk))
        args = (cq, sq_, ck, sk_, cv, sv_.reshape(B, Hkv))
    else:
        args = (dev(qc), dev(qs), dev(kc), dev(ks), dev(vc), dev(vs.reshape(B, Hkv)))
    o = torch.full((B, Hq, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_forward_fp8(*args, o, lse, causal, scale)
    torch.cuda.synchronize()
    # The bar follows the kernel's arithmetic key by key (fa_cases.fp8_bound_terms):
    # a deterministic term for probabilities small enough to flush to zero, a
    # Hoeffding term for the other keys' E4M3 rounding of P, the bf16 rounding
    # of O, and a mean-abs bar over every compared element.
    vd = oracle.dequantize_fp8(vc, vs, max(1, Nk))
    qd, kd = oracle.dequantize_fp8(qc, qs, 128), oracle.dequantize_fp8(kc, ks, 128)
    o_ref, l_ref = oracle.attention_fp8(qc, qs, kc, ks, vc, vs, scale, causal, rows=rows)
    D, R, _, _ = fp8_bound_terms(qd, kd, vd, scale, causal, rows=rows)
    bound, mean_bar = fp8_bars(D, R, o_ref)
    got = bf16_dev_to_f64(o)
    lg = lse.cpu().numpy().astype(np.float64)
    if rows is not None:  # the sampled rows of every (batch, head)
        bi, hi = np.indices(np.asarray(rows).shape[:2])
        got = got[bi[..., None], hi[..., None], rows]
        lg = lg[bi[..., None], hi[..., None], rows]
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(lg), ~fin)
    assert (got[~fin] == 0).all()
    err = np.abs(got - o_ref)
    worst = float((err / bound).max())
    lerr = float((np.abs(lg[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))).max()) if fin.any() else 0.0
    mean_err = float(err.mean()) if err.size else 0.0
    say("  fp8: O max|d|=%.3e mean|d|=%.3e (bar %.3e) worst |d|/bound=%.3f  LSE rel=%.3e" % (
        err.max(), mean_err, mean_bar, worst, lerr))
    assert worst <= 1.0, "fp8: O exceeds its element-wise bound (%.3f)" % worst
    assert mean_err <= mean_bar, "fp8: O mean-abs %.3e above its bar %.3e" % (mean_err, mean_bar)
    assert lerr <= 1e-3


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", FP8,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_forward_fp8(B, Hq, Hkv, Nq, Nk, d, causal, gpu_lib):
    check_fp8(B, Hq, Hkv, Nq, Nk, d, causal, seed=141 + Nq)


def test_forward_fp8_with_gpu_quantizer(gpu_lib):
    check_fp8(1, 8, 2, 700, 700, 128, True, seed=151, gpu_quantize=True)


def test_forward_fp8_config3_sampled_rows(gpu_lib):
    # The timed FP8 workload: the causal GQA 64/8 N=8192 d=128 prefill inputs
    # (bf16 N(0,1)) quantized per 128-row block, 64 sampled rows per head.
    case = PrefillCase(1, 64, 8, 8192, 8192, 128, True, seed=1003)
    f = oracle.bf16_bits_to_f64
    rows = np.stack([np.stack([gen.row_sample(1003, 8192, 64, salt=1000 + h) for h in range(64)])])
    check_fp8(1, 64, 8, 8192, 8192, 128, True, seed=1003, gpu_quantize=True,
              inputs=(f(case.q_bits), f(case.k_bits), f(case.v_bits)), rows=rows)


# ------------------------------------------------- reference moved after the first tile
# Inputs whose running row maximum keeps rising along the keys (K rows scaled by
# a ramp) or jumps at one late key (a key aligned with every query of its head
# group, ~40 above the other logits in base-2 units). The kernels' vector phase
# then meets tiles, after a row's first one, whose probabilities against the
# current reference exceed the lazy-rescale slack: it must take the tile's max,
# move the reference, rescale O and the row sum, and recompute the tile.
# Rows become peaky, with |O| up to single |V| entries, where bf16 rounding of
# O alone can exceed the absolute 1e-2 bar: O is held to the element-wise
# bound of the bf16 arithmetic, as for the wide-score case above.

def _ramped(k, lo=0.5, hi=4.0):
    n = k.shape[-2]
    return k * (lo + (hi - lo) * np.arange(n) / max(1, n - 1))[:, None]


def _spiked(q, k, key, scale, logit2=40.0):
    """q rows of each head group pulled toward one direction u (the group's
    first query row), and key `key` of the group set to t*u with
    t*|u|^2*scale*log2(e) = logit2."""
    q, k = q.copy(), k.copy()
    B, Hkv = k.shape[:2]
    G = q.shape[1] // Hkv
    for b in range(B):
        for g in range(Hkv):
            u = q[b, g * G, 0].copy()
            q[b, g * G:(g + 1) * G] = u + 0.25 * q[b, g * G:(g + 1) * G]
            k[b, g, key] = logit2 / (float(u @ u) * scale * math.log2(math.e)) * u
    return q, k


@pytest.mark.parametrize("causal", [True, False])
def test_rising_scores(causal, gpu_lib):
    case = PrefillCase(1, 8, 2, 1000, 1000, 128, causal, seed=161)
    case.k_bits = f64_to_bf16_bits(_ramped(oracle.bf16_bits_to_f64(case.k_bits)))
    check_prefill(case, what="rising scores", bf16_bound=True)


def test_rising_scores_window(gpu_lib):
    case = PrefillCase(1, 4, 2, 900, 900, 64, True, seed=162, window=(300, -1))
    case.k_bits = f64_to_bf16_bits(_ramped(oracle.bf16_bits_to_f64(case.k_bits)))
    check_prefill(case, what="rising scores, window", bf16_bound=True)


@pytest.mark.parametrize("causal", [True, False])
def test_late_spike(causal, gpu_lib):
    case = PrefillCase(1, 8, 2, 700, 700, 128, causal, seed=163)
    q, k = _spiked(oracle.bf16_bits_to_f64(case.q_bits), oracle.bf16_bits_to_f64(case.k_bits), 555, case.scale)
    case.q_bits, case.k_bits = f64_to_bf16_bits(q), f64_to_bf16_bits(k)
    check_prefill(case, what="late spike", bf16_bound=True)


def test_fp8_rising_scores(gpu_lib):
    q, k, v = _fp8_inputs(171, 1, 8, 2, 1000, 1000, 128)
    check_fp8(1, 8, 2, 1000, 1000, 128, True, seed=171, inputs=(q, _ramped(k), v))


def test_fp8_late_spike(gpu_lib):
    q, k, v = _fp8_inputs(172, 1, 8, 2, 700, 700, 128)
    q, k = _spiked(q, k, 555, float(np.float32(1.0 / np.sqrt(128))))
    check_fp8(1, 8, 2, 700, 700, 128, False, seed=172, inputs=(q, k, v))
