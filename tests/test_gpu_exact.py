"""GPU tests whose expected result is exact (bit for bit), pinning the mask and
block-table logic, plus structural invariants (determinism, paging and GQA
are storage/sharing only, decode is the last row of a causal prefill)."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
from fa_cases import DecodeCase, PrefillCase, bf16_dev_to_f64, compare, say, to_dev_bf16

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
