"""GPU tests whose expected result is exact (bit for bit), pinning the mask and
block-table logic, plus structural invariants (determinism, paging and GQA
are storage/sharing only, decode is the last row of a causal prefill)."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
from fa_cases import DecodeCase, PagedPrefillCase, PrefillCase, bf16_dev_to_f64, compare, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Nq,Nk,causal,d", [(300, 300, True, 128), (77, 333, True, 128),
                                            (130, 130, False, 64), (1, 515, True, 128)])
def test_zero_query_counts_visible_keys(Nq, Nk, causal, d, gpu_lib):
    """Q = 0: every visible logit is 0, so exp(LSE) is exactly the number of
    visible keys and O the mean of the visible values."""
    say("zero-q Nq=%d Nk=%d causal=%d d=%d" % (Nq, Nk, causal, d))
    case = PrefillCase(1, 4, 2, Nq, Nk, d, causal, seed=21)
    zq = np.zeros_like(case.q_bits)
    o, lse = case.run_gpu(q_bits=zq)
    l = lse.cpu().numpy().astype(np.float64)
    i = np.arange(Nq)
    count = np.minimum(Nk, i + 1 + Nk - Nq) if causal else np.full(Nq, Nk)
    assert np.array_equal(np.rint(np.exp(l[0])), np.broadcast_to(count, l[0].shape))
    o_ref, l_ref = case.oracle(q_bits=zq)
    compare(bf16_dev_to_f64(o), l, o_ref, l_ref, "zero-q")


def test_causal_row_zero_bit_equals_first_value(gpu_lib):
    case = PrefillCase(2, 8, 2, 200, 200, 128, True, seed=22)
    o, lse = case.run_gpu()
    ob = o.view(torch.int16).cpu().numpy().view(np.uint16)
    v = case.v_bits
    for h in range(8):
        assert np.array_equal(ob[:, h, 0], v[:, h // 4, 0]), h
    q = oracle.bf16_bits_to_f64(case.q_bits[:, :, 0])
    k = oracle.bf16_bits_to_f64(np.repeat(case.k_bits[:, :, 0], 4, axis=1))
    np.testing.assert_allclose(lse.cpu().numpy()[:, :, 0], case.scale * (q * k).sum(-1), rtol=2e-6, atol=2e-6)


def test_determinism_prefill(gpu_lib):
    case = PrefillCase(2, 16, 4, 700, 700, 128, True, seed=23)
    o1, l1 = case.run_gpu()
    o2, l2 = case.run_gpu()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_full_size_launches_repeat_bit_for_bit(gpu_lib):
    """Every timed launch at its full size, run several times in a row on the
    same inputs, must give the same bits each time: the kernels have no
    atomics and fixed summation orders, so any difference would come from a
    race (an LDS stage overwritten while still read, a copy not waited for)
    that the sampled parity checks might miss. The 8K causal GQA inputs feed
    the prefill, its window and block-sparse variants, the FP8 prefill and the
    backward; a paged chunked prefill (8 sequences, 1024-token chunks over
    8192-token caches in permuted pages) covers the paged kernel."""
    import exact_attention_03_amd as fa
    B, Hq, Hkv, N, d = 1, 64, 8, 8192, 128
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q = to_dev_bf16(gen.normal_bf16(1003, gen.STREAM_Q, (B, Hq, N, d)))
    k = to_dev_bf16(gen.normal_bf16(1003, gen.STREAM_K, (B, Hkv, N, d)))
    v = to_dev_bf16(gen.normal_bf16(1003, gen.STREAM_V, (B, Hkv, N, d)))
    do = to_dev_bf16(gen.normal_bf16(1003, gen.STREAM_DO, (B, Hq, N, d)))

    def same(runs, what):
        first = runs[0]
        for n, other in enumerate(runs[1:], 1):
            for a, b in zip(first, other):
                x, y = (a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else (a, b)
                assert torch.equal(x, y), "%s: run %d differs from run 0" % (what, n)

    def forward(launch, reps=4):
        runs = []
        for _ in range(reps):
            o = torch.full_like(q, float("nan"))
            lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda")
            launch(o, lse)
            runs.append((o, lse))
        torch.cuda.synchronize()
        return runs

    say("full-size repeat runs: prefill, window, block-sparse, FP8, backward, paged prefill")
    same(forward(lambda o, l: fa.fa_forward(q, k, v, o, l, True, scale)), "prefill")
    same(forward(lambda o, l: fa.fa_forward_window(q, k, v, o, l, True, 4096, -1, scale), 2), "window")
    mask = torch.from_numpy(gen.local_global_block_mask(64, 64, 16, 1)[None, None].copy()).cuda()
    same(forward(lambda o, l: fa.fa_forward_block_sparse(q, k, v, o, l, True, mask, scale), 2), "block-sparse")
    cq, ck, cv = (torch.empty(t.shape, dtype=torch.uint8, device="cuda") for t in (q, k, v))
    sq = torch.empty((B, Hq, N // 128), device="cuda")
    sk = torch.empty((B, Hkv, N // 128), device="cuda")
    sv = torch.empty((B, Hkv, 1), device="cuda")
    fa.fa_quantize_fp8(q, cq, sq, 128)
    fa.fa_quantize_fp8(k, ck, sk, 128)
    fa.fa_quantize_fp8(v, cv, sv, N)
    same(forward(lambda o, l: fa.fa_forward_fp8(cq, sq, ck, sk, cv, sv.reshape(B, Hkv), o, l, True, scale), 3),
         "FP8 prefill")
    o, lse = forward(lambda o, l: fa.fa_forward(q, k, v, o, l, True, scale), 1)[0]
    ws = torch.empty(fa.fa_backward_workspace_size(B, Hq, N), dtype=torch.uint8, device="cuda")
    grads = []
    for _ in range(2):
        g = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan")))
        fa.fa_backward(q, k, v, o, lse, do, g[0], g[1], g[2], True, scale, ws)
        grads.append(g)
    torch.cuda.synchronize()
    same(grads, "backward")
    # paged chunked prefill: 8 sequences, 8192 cached tokens each, the last 1024 as queries
    S, L, C = 8, 8192, 1024
    pages = S * L // 16
    kp = to_dev_bf16(gen.normal_bf16(1006, gen.STREAM_K, (pages, Hkv, 16, d)))
    vp = to_dev_bf16(gen.normal_bf16(1006, gen.STREAM_V, (pages, Hkv, 16, d)))
    qp = to_dev_bf16(gen.normal_bf16(1006, gen.STREAM_Q, (S * C, Hq, d)))
    table = torch.from_numpy(np.random.default_rng(5).permutation(pages).astype(np.int32).reshape(S, L // 16)).cuda()
    lens = torch.full((S,), L, dtype=torch.int32, device="cuda")
    cu = torch.from_numpy(np.arange(0, (S + 1) * C, C, dtype=np.int32)).cuda()
    pruns = []
    for _ in range(3):
        op = torch.full_like(qp, float("nan"))
        lp = torch.full((S * C, Hq), float("nan"), dtype=torch.float32, device="cuda")
        fa.fa_paged_prefill(qp, kp, vp, table, lens, cu, op, lp, C, True, scale)
        pruns.append((op, lp))
    torch.cuda.synchronize()
    same(pruns, "paged prefill")


def test_determinism_decode(gpu_lib):
    case = DecodeCase(6, 64, 8, 128, seed=24, len_lo=1, len_hi=5000)
    o1, l1 = case.run_gpu()
    o2, l2 = case.run_gpu()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_one_hot_key_selects_value_through_block_table(gpu_lib):
    """One key per (sequence, K/V head) gets a logit >= 110 above every other
    key; its V row holds an exact integer code of its token index. exp(-110)
    underflows to 0 in float32, so O must equal the code bit for bit: any
    wrong page or slot lookup picks another row."""
    lens = [1, 15, 16, 17, 1024, 1025, 3000, 4096]
    d, Hq, Hkv = 128, 16, 2
    base = DecodeCase(len(lens), Hq, Hkv, d, seed=25, seq_lens=lens)
    r = np.random.default_rng(5)
    one = np.uint16(0x3F80)       # bf16 1.0
    big = np.uint16(0x4220)       # bf16 40.0
    for trial in range(4):
        kb = np.zeros_like(base.k_bits)
        vb = base.v_bits.copy()
        qb = np.zeros_like(base.q_bits)
        qb[:, :, 0] = big                       # q . k* = 1600, scaled ~141
        want = np.zeros((len(lens), Hkv), dtype=np.int64)
        for b, L in enumerate(lens):
            for g in range(Hkv):
                t = [0, L - 1, (L - 1) // 2, int(r.integers(0, L))][trial]
                want[b, g] = t
                page, slot = base.table[b, t // 16], t % 16
                kb[page, g, slot, 0] = big
                code = np.array([t % 128, t // 128], dtype=np.float32)
                vb[page, g, slot, :2] = (code.view(np.uint32) >> 16).astype(np.uint16)
                vb[page, g, slot, 2:] = one
        o, lse = base.run_gpu(q_bits=qb, k_bits=kb, v_bits=vb)
        of = bf16_dev_to_f64(o)
        for b in range(len(lens)):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                got = of[b, h]
                assert got[0] == want[b, g] % 128 and got[1] == want[b, g] // 128, (trial, b, h, got[:2])
                assert (got[2:] == 1.0).all()


def test_page_tails_and_unused_pages_never_affect_output(gpu_lib):
    lens = [3, 16, 31, 1030, 2049]
    case = DecodeCase(len(lens), 8, 2, 128, seed=26, seq_lens=lens)
    o1, l1 = case.run_gpu()
    kb, vb = case.k_bits.copy(), case.v_bits.copy()
    for b, L in enumerate(lens):
        last = case.table[b, (L - 1) // 16]
        tail = L % 16
        if tail:
            kb[last, :, tail:, :] = 0x7FC0     # NaN
            vb[last, :, tail:, :] = 0x7FC0
    o2, l2 = case.run_gpu(k_bits=kb, v_bits=vb)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    for b, L in enumerate(lens):
        last = case.table[b, (L - 1) // 16]
        tail = L % 16
        if tail:
            kb[last, :, tail:, :] = 0x7F00     # 1.7e38
            vb[last, :, tail:, :] = 0xFF00
    o3, l3 = case.run_gpu(k_bits=kb, v_bits=vb)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)


def test_paging_is_storage_only(gpu_lib):
    """Moving pages to other pool slots (and rewriting the table) changes no bit."""
    lens = [100, 2000, 1500]
    case = DecodeCase(len(lens), 16, 2, 128, seed=27, seq_lens=lens)
    o1, l1 = case.run_gpu()
    P = case.num_pages
    new_of = np.random.default_rng(9).permutation(P)
    kb = np.empty_like(case.k_bits); vb = np.empty_like(case.v_bits)
    kb[new_of] = case.k_bits; vb[new_of] = case.v_bits
    table = np.where(case.table >= 0, new_of[np.maximum(case.table, 0)], -1).astype(np.int32)
    o2, l2 = case.run_gpu(k_bits=kb, v_bits=vb, table=table)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_equals_last_row_of_causal_prefill(gpu_lib):
    import exact_attention_03_amd as fa
    lens = [1, 40, 1500]
    Hq, Hkv, d = 16, 4, 128
    case = DecodeCase(len(lens), Hq, Hkv, d, seed=28, seq_lens=lens)
    o, lse = case.run_gpu()
    for b, L in enumerate(lens):
        kc = oracle.gather_pages(case.k_bits, case.table[b], L, 16)[None]   # [1, Hkv, L, d] bits
        vc = oracle.gather_pages(case.v_bits, case.table[b], L, 16)[None]
        q = to_dev_bf16(case.q_bits[b][None, :, None, :].copy())
        of = torch.empty((1, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
        lf = torch.empty((1, Hq, 1), dtype=torch.float32, device="cuda")
        fa.fa_forward(q, to_dev_bf16(kc.copy()), to_dev_bf16(vc.copy()), of, lf, True, case.scale)
        torch.cuda.synchronize()
        a = bf16_dev_to_f64(o[b]); c = bf16_dev_to_f64(of[0, :, 0])
        assert np.abs(a - c).max() <= 1e-2
        assert np.abs(lse[b].cpu().numpy() - lf[0, :, 0].cpu().numpy()).max() <= 1e-3 * max(1.0, float(lse[b].abs().max()))


def test_gqa_equals_mha_with_repeated_heads(gpu_lib):
    case = PrefillCase(1, 16, 2, 333, 333, 128, True, seed=29)
    o1, l1 = case.run_gpu()
    mha = PrefillCase(1, 16, 16, 333, 333, 128, True, seed=29)
    kr = np.repeat(case.k_bits, 8, axis=1)
    vr = np.repeat(case.v_bits, 8, axis=1)
    o2, l2 = mha.run_gpu(q_bits=case.q_bits, k_bits=kr, v_bits=vr)
    assert np.abs(bf16_dev_to_f64(o1) - bf16_dev_to_f64(o2)).max() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


# ---- exact visible-key counts for the window, block-sparse and paged paths ----
# With Q = 0 every visible logit is exactly 0, so the kernel's row sum is the
# number of visible keys (an integer, exact in float32) and rint(exp(LSE))
# must equal the count written out below from the mask's definition: any
# off-by-one at a window edge, a block edge or a page boundary changes it.

def window_counts(Nq, Nk, causal, window):
    """Keys visible from each query row: row i sits at key position
    p = i + Nk - Nq and sees p - left <= j <= p + right (-1 = unbounded;
    causal caps the right edge at p), clipped to [0, Nk)."""
    p = np.arange(Nq) + (Nk - Nq)
    left, right = window if window is not None else (-1, -1)
    lo = np.maximum(0, p - left) if left >= 0 else np.zeros(Nq, dtype=np.int64)
    hi = np.full(Nq, Nk - 1)
    if right >= 0:
        hi = np.minimum(hi, p + right)
    if causal:
        hi = np.minimum(hi, p)
    return np.maximum(0, hi - lo + 1)


def block_counts(mask_bh, Nq, Nk, causal, block=128):
    """Keys visible from each query row under a block mask [nqb, nkb]: the
    keys of every set key block of the row's query block, causally capped."""
    p = np.arange(Nq) + (Nk - Nq)
    cnt = np.zeros(Nq, dtype=np.int64)
    for kb in range(mask_bh.shape[1]):
        k0, k1 = kb * block, min(Nk, (kb + 1) * block)
        hi = np.minimum(k1 - 1, p) if causal else np.full(Nq, k1 - 1)
        n = np.maximum(0, hi - k0 + 1)
        cnt += np.where(mask_bh[np.arange(Nq) // block, kb] != 0, n, 0)
    return cnt


def assert_counts(lse, counts, what):
    """lse [..., rows] (float32 on the device), counts broadcastable to it."""
    l = lse.cpu().numpy().astype(np.float64)
    c = np.broadcast_to(counts, l.shape)
    got = np.where(np.isneginf(l), 0, np.rint(np.exp(np.where(np.isneginf(l), 0.0, l))))
    bad = got != c
    say("  %s: %d rows, counts %d..%d, %d mismatches" % (what, c.size, c.min(), c.max(), int(bad.sum())))
    assert not bad.any(), "%s: first mismatch at %s: got %d want %d" % (
        what, np.argwhere(bad)[0], got[bad][0], c[bad][0])
    assert np.array_equal(np.isneginf(l), c == 0), what + ": rows without keys must have LSE = -inf"


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,win", [
    (1, 8, 1, 8192, 8192, 128, True, (4096, -1)),     # the timed window: 4097 keys, G=8 packing
    (1, 4, 2, 3000, 3000, 128, False, (1000, 700)),   # two-sided
    (2, 4, 2, 900, 2000, 64, True, (511, -1)),        # Nq < Nk, d=64
    (1, 8, 8, 1000, 1000, 128, False, (-1, 129)),     # right edge only, G=1
    (1, 4, 1, 700, 700, 128, True, (127, -1)),        # window edge on a tile edge
])
def test_window_zero_query_counts(B, Hq, Hkv, Nq, Nk, d, causal, win, gpu_lib):
    say("zero-q window %s B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d" % (win, B, Hq, Hkv, Nq, Nk, d, causal))
    case = PrefillCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=201, window=win)
    zq = np.zeros_like(case.q_bits)
    o, lse = case.run_gpu(q_bits=zq)
    assert_counts(lse, window_counts(Nq, Nk, causal, win), "window %s" % (win,))
    rows = gen.row_sample(201, Nq, min(Nq, 64))
    o_ref, l_ref = case.oracle(rows=rows, q_bits=zq)
    compare(bf16_dev_to_f64(o)[:, :, rows], lse.cpu().numpy().astype(np.float64)[:, :, rows], o_ref, l_ref,
            "zero-q window")


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,pattern", [
    (1, 8, 1, 2000, 2000, 128, True, "random50"),     # per-head masks, G=8
    (1, 2, 2, 700, 1300, 64, False, "random30"),      # Nq != Nk, d=64, G=1
    (1, 8, 1, 8192, 8192, 128, True, "local16+global1"),  # the timed pattern
    (2, 4, 2, 513, 513, 128, True, "random60"),       # per batch, ragged
])
def test_block_sparse_zero_query_counts(B, Hq, Hkv, Nq, Nk, d, causal, pattern, gpu_lib):
    say("zero-q block-sparse %s B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d causal=%d" % (
        pattern, B, Hq, Hkv, Nq, Nk, d, causal))
    nqb, nkb = -(-Nq // 128), -(-Nk // 128)
    if pattern.startswith("random"):
        mask = gen.random_block_mask(211 + Nq, (B, Hq, nqb, nkb), int(pattern[6:]))
    else:
        mask = np.broadcast_to(gen.local_global_block_mask(nqb, nkb, 16, 1)[None, None], (B, Hq, nqb, nkb))
    case = PrefillCase(B, Hq, Hkv, Nq, Nk, d, causal, seed=211, block_mask=np.ascontiguousarray(mask))
    zq = np.zeros_like(case.q_bits)
    o, lse = case.run_gpu(q_bits=zq)
    want = np.stack([np.stack([block_counts(mask[b, h], Nq, Nk, causal) for h in range(Hq)]) for b in range(B)])
    assert_counts(lse, want, "block-sparse %s" % pattern)
    rows = gen.row_sample(211, Nq, min(Nq, 64))
    o_ref, l_ref = case.oracle(rows=rows, q_bits=zq)
    compare(bf16_dev_to_f64(o)[:, :, rows], lse.cpu().numpy().astype(np.float64)[:, :, rows], o_ref, l_ref,
            "zero-q block-sparse")


@pytest.mark.parametrize("Hq,Hkv,d,causal,window,lens,chunks", [
    (8, 1, 128, True, None, [3000, 17, 1000, 64, 4096], [1024, 5, 129, 1, 4096]),
    (16, 2, 128, True, (1023, -1), [5000, 1100, 40], [700, 1100, 40]),
    (6, 2, 128, False, (100, 50), [1000, 333], [260, 7]),
    (4, 4, 64, True, None, [77, 256, 1, 0], [30, 256, 1, 3]),
])
def test_paged_prefill_zero_query_counts(Hq, Hkv, d, causal, window, lens, chunks, gpu_lib):
    say("zero-q paged prefill window=%s Hq=%d Hkv=%d d=%d causal=%d lens=%s chunks=%s" % (
        window, Hq, Hkv, d, causal, lens, chunks))
    case = PagedPrefillCase(Hq, Hkv, d, seed=221, seq_lens=lens, q_lens=chunks, causal=causal, window=window)
    case.q_bits = np.zeros_like(case.q_bits)
    o, lse = case.run_gpu()
    want = np.concatenate([window_counts(n, L, causal, window) for L, n in zip(lens, chunks)])
    assert_counts(lse.T, want[None, :], "paged prefill window=%s" % (window,))
    o_ref, l_ref = case.oracle()
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "zero-q paged prefill")


@pytest.mark.parametrize("causal", [False, True])
def test_one_hot_key_selects_value_through_paged_prefill_table(causal, gpu_lib):
    """The decode test's recipe through the chunked prefill's page table: one
    key per (sequence, K/V head) gets a logit >= 110 above every other key and
    holds an exact integer code of its token index in V; every query row of
    the chunk must return that code bit for bit. Causally the key is placed
    where every row of the chunk sees it (at or before the chunk's first
    position)."""
    lens = [1, 15, 16, 17, 1024, 1025, 3000, 4096]
    chunks = [1, 5, 16, 17, 100, 1025, 64, 300]
    d, Hq, Hkv = 128, 16, 2
    base = PagedPrefillCase(Hq, Hkv, d, seed=231, seq_lens=lens, q_lens=chunks, causal=causal)
    r = np.random.default_rng(6)
    one = np.uint16(0x3F80)       # bf16 1.0
    big = np.uint16(0x4220)       # bf16 40.0
    q0 = np.zeros_like(base.q_bits)
    q0[:, :, 0] = big             # q . k* = 1600, scaled ~141
    k0, v0 = base.k_bits, base.v_bits
    for trial in range(4):
        kb = np.zeros_like(k0)
        vb = v0.copy()
        want = np.zeros((len(lens), Hkv), dtype=np.int64)
        for b, (L, n) in enumerate(zip(lens, chunks)):
            last = L - n if causal else L - 1        # latest key every row sees
            for g in range(Hkv):
                t = [0, last, last // 2, int(r.integers(0, last + 1))][trial]
                want[b, g] = t
                page, slot = base.table[b, t // 16], t % 16
                kb[page, g, slot, 0] = big
                code = np.array([t % 128, t // 128], dtype=np.float32)
                vb[page, g, slot, :2] = (code.view(np.uint32) >> 16).astype(np.uint16)
                vb[page, g, slot, 2:] = one
        base.q_bits, base.k_bits, base.v_bits = q0, kb, vb
        say("one-hot paged prefill causal=%d trial %d" % (causal, trial))
        o, lse = base.run_gpu()
        of = bf16_dev_to_f64(o)
        for b in range(len(lens)):
            rows = of[base.cu[b]:base.cu[b + 1]]             # [n, Hq, d]
            for h in range(Hq):
                g = h // (Hq // Hkv)
                assert (rows[:, h, 0] == want[b, g] % 128).all() and (rows[:, h, 1] == want[b, g] // 128).all(), \
                    (trial, b, h, rows[:, h, :2])
                assert (rows[:, h, 2:] == 1.0).all()
