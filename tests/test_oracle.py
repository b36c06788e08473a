"""Pins for the CPU oracle, against facts other than the oracle itself.

Each pin names the fact that fixes it:
  * a library routine (torch's scaled_dot_product_attention in float64 on the
    CPU, and scipy's logsumexp) -- special cases that reduce to them;
  * closed forms (Q = 0 gives the mean of the visible values and LSE = ln of
    the visible count; a single visible key gives that key's value and its
    scaled logit; duplicating every key adds ln 2 to LSE);
  * the invariants the pages state (softmax weights in [0, 1] summing to 1;
    paging stores the cache without changing the computation; GQA is MHA with
    shared K/V heads);
  * brute force (naive == online == split-K on tiny shapes);
  * hand-worked examples stored under tests/golden with their citation.
The last block plants plausible mistakes in copies of the oracle and checks
that some pin fails for each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def rnd(*shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def sdpa_f64(q, k, v, scale, causal):
    """torch's SDPA in float64 on the CPU, K/V heads repeated for GQA, causal
    mask given explicitly as the bottom-right lower triangle."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    kt = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
    vt = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
    mask = None
    if causal:
        mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, attn_mask=mask, scale=scale).numpy()


SHAPES = [  # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 7, 7, 4, False),
    (2, 4, 2, 13, 13, 8, True),
    (1, 8, 1, 5, 19, 16, True),       # MQA, Nq < Nk: bottom-right causal
    (2, 6, 3, 17, 9, 8, False),
    (1, 2, 2, 33, 33, 64, True),
]


def run_sdpa_pin(naive_fn, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = rnd(B, Hq, Nq, d), rnd(B, Hkv, Nk, d), rnd(B, Hkv, Nk, d)
    scale = 1.0 / np.sqrt(d)
    O, _ = naive_fn(q, k, v, scale, causal)
    return np.abs(O - sdpa_f64(q, k, v, scale, causal)).max()


@pytest.mark.parametrize("shape", SHAPES)
def test_naive_matches_torch_sdpa(shape):
    assert run_sdpa_pin(oracle.attention_naive, shape) < 1e-12


@pytest.mark.parametrize("shape", SHAPES)
def test_lse_matches_scipy_logsumexp(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = rnd(B, Hq, Nq, d), rnd(B, Hkv, Nk, d), rnd(B, Hkv, Nk, d)
    scale = 0.3
    _, lse = oracle.attention_naive(q, k, v, scale, causal)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            s = scale * np.einsum("id,jd->ij", q[b, h], k[b, h // G])
            i = np.arange(Nq)[:, None]
            j = np.arange(Nk)[None, :]
            vis = (j <= i + Nk - Nq) if causal else np.ones((Nq, Nk), bool)
            want = scipy.special.logsumexp(np.where(vis, s, -np.inf), axis=1)
            np.testing.assert_allclose(lse[b, h], want, rtol=0, atol=1e-12)


def test_p_rows_are_probability_vectors():
    q, k, v = rnd(2, 4, 21, 8), rnd(2, 2, 21, 8), rnd(2, 2, 21, 8)
    O, lse, P = oracle.attention_naive(q, k, v, 0.35, True, return_p=True)
    assert (P >= 0).all() and (P <= 1).all()
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    above = np.arange(21)[None, :] > np.arange(21)[:, None]
    assert (P[:, :, above] == 0).all()


@pytest.mark.parametrize("causal,Nq,Nk", [(False, 9, 14), (True, 9, 9), (True, 6, 15)])
def test_zero_query_gives_mean_of_visible_values(causal, Nq, Nk):
    q = np.zeros((1, 4, Nq, 8))
    k, v = rnd(1, 2, Nk, 8), rnd(1, 2, Nk, 8)
    O, lse = oracle.attention_naive(q, k, v, 0.7, causal)
    for h in range(4):
        g = h // 2
        for i in range(Nq):
            n_vis = (i + Nk - Nq + 1) if causal else Nk
            np.testing.assert_allclose(O[0, h, i], v[0, g, :n_vis].mean(0), atol=1e-13)
            assert abs(lse[0, h, i] - np.log(n_vis)) < 1e-13


def test_causal_row_zero_is_first_value():
    q, k, v = rnd(2, 3, 12, 16), rnd(2, 3, 12, 16), rnd(2, 3, 12, 16)
    O, lse = oracle.attention_naive(q, k, v, 0.25, True)
    assert np.array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-14)


def test_one_hot_logit_selects_value_row():
    d, Nk = 16, 40
    for t_star in (0, 17, 39):
        q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
        k = rnd(1, 1, Nk, d, sigma=0.01); k[0, 0, t_star, 0] = 800.0
        v = rnd(1, 1, Nk, d)
        O, lse = oracle.attention_naive(q, k, v, 1.0, False)
        np.testing.assert_allclose(O[0, 0, 0], v[0, 0, t_star], rtol=0, atol=1e-300)


def test_duplicated_keys_add_ln2():
    q, k, v = rnd(1, 2, 5, 8), rnd(1, 2, 7, 8), rnd(1, 2, 7, 8)
    O1, l1 = oracle.attention_naive(q, k, v, 0.5, False)
    O2, l2 = oracle.attention_naive(q, np.concatenate([k, k], 2), np.concatenate([v, v], 2), 0.5, False)
    np.testing.assert_allclose(O2, O1, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, np.log(2.0), atol=1e-13)


def test_key_permutation_invariance():
    q, k, v = rnd(1, 2, 6, 8), rnd(1, 1, 11, 8), rnd(1, 1, 11, 8)
    perm = np.random.default_rng(3).permutation(11)
    O1, l1 = oracle.attention_naive(q, k, v, 0.4, False)
    O2, l2 = oracle.attention_naive(q, k[:, :, perm], v[:, :, perm], 0.4, False)
    np.testing.assert_allclose(O2, O1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)


def test_gqa_equals_mha_with_repeated_heads():
    q, k, v = rnd(2, 8, 10, 8), rnd(2, 2, 10, 8), rnd(2, 2, 10, 8)
    O1, l1 = oracle.attention_naive(q, k, v, 0.4, True)
    O2, l2 = oracle.attention_naive(q, np.repeat(k, 4, 1), np.repeat(v, 4, 1), 0.4, True)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    assert [oracle.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


@pytest.mark.parametrize("tile", [1, 3, 16, 64])
@pytest.mark.parametrize("causal,Nq,Nk", [(False, 13, 29), (True, 29, 29), (True, 10, 29)])
def test_online_equals_naive(tile, causal, Nq, Nk):
    q, k, v = rnd(1, 4, Nq, 8), rnd(1, 2, Nk, 8), rnd(1, 2, Nk, 8)
    O1, l1 = oracle.attention_naive(q, k, v, 0.6, causal)
    O2, l2 = oracle.attention_online(q, k, v, 0.6, causal, tile=min(tile, Nk))
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


@pytest.mark.parametrize("bounds", [[0, 29], [0, 10, 29], [0, 0, 5, 5, 29, 29], [0, 1, 2, 3, 28, 29]])
def test_split_combine_equals_naive(bounds):
    q, k, v = rnd(1, 4, 12, 8), rnd(1, 2, 29, 8), rnd(1, 2, 29, 8)
    O1, l1 = oracle.attention_naive(q, k, v, 0.6, True)
    O2, l2 = oracle.attention_split(q, k, v, 0.6, True, bounds, tile=4)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_fully_masked_rows_and_empty_keys():
    q, k, v = rnd(1, 1, 8, 4), rnd(1, 1, 3, 4), rnd(1, 1, 3, 4)
    O, lse = oracle.attention_naive(q, k, v, 1.0, True)     # Nk < Nq: rows 0..4 see nothing
    assert (O[0, 0, :5] == 0).all() and np.isneginf(lse[0, 0, :5]).all()
    assert np.isfinite(lse[0, 0, 5:]).all()
    O2, l2 = oracle.attention_online(q, k, v, 1.0, True, tile=2)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    assert np.isneginf(l2[0, 0, :5]).all()
    O3, l3 = oracle.attention_naive(q, k[:, :, :0], v[:, :, :0], 1.0, False)
    assert (O3 == 0).all() and np.isneginf(l3).all()


def test_rows_subset_matches_full():
    q, k, v = rnd(1, 4, 40, 8), rnd(1, 2, 40, 8), rnd(1, 2, 40, 8)
    O, lse = oracle.attention_naive(q, k, v, 0.5, True)
    rows = np.array([[[0, 7, 39], [1, 2, 3], [38, 39, 0], [5, 5, 5]]])
    Os, ls = oracle.attention_naive(q, k, v, 0.5, True, rows=rows)
    for h in range(4):
        np.testing.assert_array_equal(Os[0, h], O[0, h, rows[0, h]])
        np.testing.assert_array_equal(ls[0, h], lse[0, h, rows[0, h]])


def make_paged(seed_rng, B, Hkv, d, lens, ps=16, extra_pages=3):
    npages = [(L + ps - 1) // ps for L in lens]
    total = sum(npages) + extra_pages
    perm = seed_rng.permutation(total)
    maxp = max(npages) + 2
    table = np.full((B, maxp), -1, np.int64)
    c = 0
    for b in range(B):
        table[b, :npages[b]] = perm[c:c + npages[b]]
        c += npages[b]
    kp = seed_rng.standard_normal((total, Hkv, ps, d))
    vp = seed_rng.standard_normal((total, Hkv, ps, d))
    return kp, vp, table


def test_paged_decode_equals_contiguous_and_causal_last_row():
    r = np.random.default_rng(9)
    lens = [1, 16, 17, 50]
    B, Hq, Hkv, d = 4, 6, 2, 8
    kp, vp, table = make_paged(r, B, Hkv, d, lens)
    q = r.standard_normal((B, Hq, d))
    O, lse = oracle.paged_decode(q, kp, vp, table, lens, 0.3)
    for b, L in enumerate(lens):
        # contiguous cache assembled by direct indexing, token by token
        kc = np.stack([kp[table[b, t // 16], :, t % 16, :] for t in range(L)], 1)
        vc = np.stack([vp[table[b, t // 16], :, t % 16, :] for t in range(L)], 1)
        o2, l2 = oracle.attention_naive(q[b][None, :, None, :], kc[None], vc[None], 0.3, False)
        np.testing.assert_allclose(O[b], o2[0, :, 0], atol=1e-13)
        # the decode token is the last row of a causal prefill over the same cache
        qq = r.standard_normal((1, Hq, L, d)); qq[0, :, L - 1] = q[b]
        o3, l3 = oracle.attention_naive(qq, kc[None], vc[None], 0.3, True)
        np.testing.assert_allclose(O[b], o3[0, :, L - 1], atol=1e-13)
        np.testing.assert_allclose(lse[b], l3[0, :, L - 1], atol=1e-13)


def test_paged_decode_ignores_page_placement_and_tail_slots():
    r = np.random.default_rng(10)
    lens = [5, 33]
    kp, vp, table = make_paged(r, 2, 1, 4, lens, extra_pages=0)
    q = r.standard_normal((2, 2, 4))
    O, lse = oracle.paged_decode(q, kp, vp, table, lens, 0.5)
    # move every page to a new slot of a permuted pool and rewrite the table
    P = kp.shape[0]
    new_of = np.random.default_rng(11).permutation(P)
    kp2 = np.empty_like(kp); vp2 = np.empty_like(vp)
    kp2[new_of] = kp; vp2[new_of] = vp
    table2 = np.where(table >= 0, new_of[np.maximum(table, 0)], -1)
    # poison the slots past each sequence's end and the unused pages
    for b, L in enumerate(lens):
        last = table2[b, (L - 1) // 16]
        kp2[last, :, L % 16 or 16:, :] = np.nan
        vp2[last, :, L % 16 or 16:, :] = np.nan
    O2, l2 = oracle.paged_decode(q, kp2, vp2, table2, lens, 0.5)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(l2, lse, atol=1e-14)


# ---- paged prefill (chunks of new queries against a paged cache) ----

def _paged_prefill_case(seed, lens, chunks, Hq=4, Hkv=2, d=8):
    r = np.random.default_rng(seed)
    kp, vp, table = make_paged(r, len(lens), Hkv, d, lens)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = r.standard_normal((int(cu[-1]), Hq, d))
    return r, kp, vp, table, cu, q


def _contiguous(kp, table, b, L):
    return np.stack([kp[table[b, t // 16], :, t % 16, :] for t in range(L)], 1) if L else \
        np.zeros((kp.shape[1], 0, kp.shape[3]))


def test_paged_prefill_full_chunk_equals_contiguous_causal_prefill():
    # A chunk covering the whole sequence is an ordinary causal prefill of the
    # gathered cache (cache assembled token by token, not with gather_pages).
    lens = [1, 16, 40, 70]
    r, kp, vp, table, cu, q = _paged_prefill_case(21, lens, lens)
    O, lse = oracle.paged_prefill(q, kp, vp, table, lens, cu, 0.4, True)
    for b, L in enumerate(lens):
        kc, vc = _contiguous(kp, table, b, L), _contiguous(vp, table, b, L)
        qb = np.transpose(q[cu[b]:cu[b + 1]], (1, 0, 2))[None]
        o2, l2 = oracle.attention_naive(qb, kc[None], vc[None], 0.4, True)
        np.testing.assert_allclose(O[cu[b]:cu[b + 1]], np.transpose(o2[0], (1, 0, 2)), atol=1e-13)
        np.testing.assert_allclose(lse[cu[b]:cu[b + 1]], l2[0].T, atol=1e-13)


def test_paged_prefill_one_token_chunk_is_decode():
    lens = [3, 17, 33]
    r, kp, vp, table, cu, q = _paged_prefill_case(22, lens, [1, 1, 1])
    for causal in (True, False):
        O, lse = oracle.paged_prefill(q, kp, vp, table, lens, cu, 0.7, causal)
        O2, l2 = oracle.paged_decode(q, kp, vp, table, lens, 0.7)
        np.testing.assert_allclose(O, O2, atol=1e-13)
        np.testing.assert_allclose(lse, l2, atol=1e-13)


def test_paged_prefill_chunks_compose():
    # Bottom-right alignment: the last rows of one chunk over L keys equal a
    # second, shorter chunk over the same L keys, and the first rows equal a
    # chunk over only the first L - (n - a) keys.
    L, n, a = 45, 20, 8
    r, kp, vp, table, cu, q = _paged_prefill_case(23, [L], [n])
    O, lse = oracle.paged_prefill(q, kp, vp, table, [L], cu, 0.5, True)
    Ot, lt = oracle.paged_prefill(q[a:], kp, vp, table, [L], np.array([0, n - a]), 0.5, True)
    np.testing.assert_allclose(O[a:], Ot, atol=1e-13)
    np.testing.assert_allclose(lse[a:], lt, atol=1e-13)
    Oh, lh = oracle.paged_prefill(q[:a], kp, vp, table, [L - (n - a)], np.array([0, a]), 0.5, True)
    np.testing.assert_allclose(O[:a], Oh, atol=1e-13)
    np.testing.assert_allclose(lse[:a], lh, atol=1e-13)


def test_paged_prefill_ignores_page_placement_and_handles_empty():
    lens = [0, 5, 33]
    r, kp, vp, table, cu, q = _paged_prefill_case(24, lens, [3, 5, 0])
    O, lse = oracle.paged_prefill(q, kp, vp, table, lens, cu, 0.5, True)
    # sequence 0 has no keys: O = 0, LSE = -inf
    assert np.all(O[0:3] == 0) and np.all(lse[0:3] == -np.inf)
    P = kp.shape[0]
    new_of = np.random.default_rng(25).permutation(P)
    kp2 = np.empty_like(kp); vp2 = np.empty_like(vp)
    kp2[new_of] = kp; vp2[new_of] = vp
    table2 = np.where(table >= 0, new_of[np.maximum(table, 0)], -1)
    O2, l2 = oracle.paged_prefill(q, kp2, vp2, table2, lens, cu, 0.5, True)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(l2, lse, atol=1e-14)


def test_paged_prefill_detects_top_left_alignment():
    # Planted mistake: a top-left causal mask (query i sees keys j <= i) for a
    # chunk shorter than its cache differs from the oracle's result.
    L, n = 30, 6
    r, kp, vp, table, cu, q = _paged_prefill_case(26, [L], [n])
    O, _ = oracle.paged_prefill(q, kp, vp, table, [L], cu, 0.5, True)
    kc, vc = _contiguous(kp, table, 0, L), _contiguous(vp, table, 0, L)
    qb = np.transpose(q, (1, 0, 2))[None]
    s = np.einsum("hid,hjd->hij", qb[0], kc[np.repeat(np.arange(2), 2)]) * 0.5
    s = np.where(np.arange(L)[None, None, :] <= np.arange(n)[None, :, None], s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True)); p /= p.sum(-1, keepdims=True)
    wrong = np.einsum("hij,hjd->hid", p, vc[np.repeat(np.arange(2), 2)])
    assert np.abs(np.transpose(wrong, (1, 0, 2)) - O).max() > 1e-3


def _windowed_rows_brute(q, kc, vc, n, L, scale, causal, left, right):
    # Row by row from the window's definition: query i of a chunk of n sits at
    # key position p = i + L - n and sees key j in [0, L) iff j >= p - left
    # (left >= 0), j <= p + right (right >= 0) and j <= p (causal).
    Hq, Hkv = q.shape[1], kc.shape[0]
    O = np.zeros((n, Hq, q.shape[2]))
    lse = np.full((n, Hq), -np.inf)
    for i in range(n):
        pos = i + L - n
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [j for j in range(L) if (left < 0 or j >= pos - left) and (right < 0 or j <= pos + right)
                    and (not causal or j <= pos)]
            if not keys:
                continue
            s = [scale * float(np.dot(q[i, h], kc[g, j])) for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            O[i, h] = sum(wj * vc[g, j] for wj, j in zip(w, keys)) / tot
            lse[i, h] = m + math.log(tot)
    return O, lse


@pytest.mark.parametrize("causal, left, right", [(True, 7, -1), (True, 0, -1), (False, 5, 3), (False, -1, 2),
                                                 (True, 40, 9), (False, 3, 0)])
def test_paged_prefill_window_matches_brute_force(causal, left, right):
    # The gathered cache is assembled token by token; rows with an empty window
    # (n > L with a tight window) come out O = 0, LSE = -inf.
    lens, chunks = [0, 9, 33, 50], [2, 9, 12, 1]
    r, kp, vp, table, cu, q = _paged_prefill_case(27, lens, chunks)
    O, lse = oracle.paged_prefill(q, kp, vp, table, lens, cu, 0.45, causal, window=(left, right))
    for b, (L, n) in enumerate(zip(lens, chunks)):
        kc, vc = _contiguous(kp, table, b, L), _contiguous(vp, table, b, L)
        Ob, lb = _windowed_rows_brute(q[cu[b]:cu[b + 1]], kc, vc, n, L, 0.45, causal, left, right)
        np.testing.assert_allclose(O[cu[b]:cu[b + 1]], Ob, atol=1e-13)
        np.testing.assert_allclose(lse[cu[b]:cu[b + 1]], lb, atol=1e-13)


def test_paged_prefill_window_last_row_is_decode_over_recent_tokens():
    # With causal and left bound w, the chunk's last query sees exactly the
    # last w + 1 tokens: a decode over a cache holding only those.
    L, n, w = 70, 10, 20
    r, kp, vp, table, cu, q = _paged_prefill_case(28, [L], [n])
    O, lse = oracle.paged_prefill(q, kp, vp, table, [L], cu, 0.5, True, window=(w, -1))
    kc, vc = _contiguous(kp, table, 0, L)[:, L - w - 1:], _contiguous(vp, table, 0, L)[:, L - w - 1:]
    kp2 = np.zeros((3, kc.shape[0], 16, kc.shape[2])); vp2 = np.zeros_like(kp2)
    for t in range(w + 1):
        kp2[t // 16, :, t % 16] = kc[:, t]
        vp2[t // 16, :, t % 16] = vc[:, t]
    Od, ld = oracle.paged_decode(q[n - 1:n], kp2, vp2, np.array([[0, 1, 2]]), [w + 1], 0.5)
    np.testing.assert_allclose(O[n - 1], Od[0], atol=1e-13)
    np.testing.assert_allclose(lse[n - 1], ld[0], atol=1e-13)


def test_paged_prefill_window_detects_off_by_one_left_bound():
    # Planted mistake: a left bound one key too tight (j > p - left) differs.
    lens, chunks = [33], [12]
    r, kp, vp, table, cu, q = _paged_prefill_case(29, lens, chunks)
    O, _ = oracle.paged_prefill(q, kp, vp, table, lens, cu, 0.45, True, window=(6, -1))
    kc, vc = _contiguous(kp, table, 0, 33), _contiguous(vp, table, 0, 33)
    wrong, _ = _windowed_rows_brute(q, kc, vc, 12, 33, 0.45, True, 5, -1)
    assert np.abs(wrong - O).max() > 1e-3


def test_bf16_decode_exact():
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0x0001, 0xC2F7], dtype=np.uint16)
    want = [0.0, 1.0, -1.0, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41, -123.5]
    assert oracle.bf16_bits_to_f64(bits).tolist() == want


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", load_golden("hand_examples.json")["cases"], ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    O, lse = oracle.attention_naive(q, k, v, case["scale"], case["causal"])
    np.testing.assert_allclose(O, np.array(case["O"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(case["LSE"]), rtol=0, atol=1e-14)


# ---- planted mistakes: each copy of the oracle must fail at least one pin ----

def _mutant(kind):
    def fn(q, k, v, scale, causal):
        if kind == "scale_inverted":
            return oracle.attention_naive(q, k, v, 1.0 / scale, causal)
        if kind == "causal_strict":          # j < i instead of j <= i
            return _strict(q, k, v, scale) if causal else oracle.attention_naive(q, k, v, scale, causal)
        if kind == "gqa_modulo":             # head h -> h % Hkv instead of h // G
            Hq, Hkv = q.shape[1], k.shape[1]
            idx = [h % Hkv for h in range(Hq)]
            return oracle.attention_naive(q, k[:, idx], v[:, idx], scale, causal)
        if kind == "k_swapped_with_v":
            return oracle.attention_naive(q, v, k, scale, causal)
        if kind == "top_left_causal":        # mask aligned to the top-left corner
            return _top_left(q, k, v, scale, causal)
        raise AssertionError(kind)
    return fn


def _strict(q, k, v, scale):
    B, Hq, Nq, d = q.shape
    Nk = k.shape[2]
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    for i in range(Nq):
        n = i + Nk - Nq          # one key fewer than the correct mask
        if n <= 0:
            L[:, :, i] = -np.inf
            continue
        o, l = oracle.attention_naive(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], scale, False)
        O[:, :, i] = o[:, :, 0]
        L[:, :, i] = l[:, :, 0]
    return O, L


def _top_left(q, k, v, scale, causal):
    if not causal:
        return oracle.attention_naive(q, k, v, scale, causal)
    Nq, Nk = q.shape[2], k.shape[2]
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    for i in range(Nq):
        n = min(i + 1, Nk)
        o, l = oracle.attention_naive(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], scale, False)
        O[:, :, i] = o[:, :, 0]
        L[:, :, i] = l[:, :, 0]
    return O, L


@pytest.mark.parametrize("kind", ["scale_inverted", "causal_strict", "gqa_modulo",
                                  "k_swapped_with_v", "top_left_causal"])
def test_planted_mistakes_are_caught(kind):
    fn = _mutant(kind)
    worst = max(run_sdpa_pin(fn, s) for s in SHAPES)
    assert worst > 1e-6, kind



# ---- sliding window ----

def _qkv(seed, B, Hq, Hkv, Nq, Nk, d):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, Nq, d)), r.standard_normal((B, Hkv, Nk, d)),
            r.standard_normal((B, Hkv, Nk, d)))


def test_window_unbounded_is_plain_attention():
    q, k, v = _qkv(51, 1, 4, 2, 30, 50, 8)
    for causal in (False, True):
        o, l = oracle.attention_naive(q, k, v, 0.3, causal)
        o2, l2 = oracle.attention_naive(q, k, v, 0.3, causal, window=(-1, -1))
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(l, l2)
    # a right window of 0 is the causal mask
    o, l = oracle.attention_naive(q, k, v, 0.3, True)
    o2, l2 = oracle.attention_naive(q, k, v, 0.3, False, window=(-1, 0))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_window_zero_selects_own_position():
    # left = 0 with causal: query i sees only key p = i + Nk - Nq, so O = V[p]
    # and LSE = scale * q_i . k_p (closed form).
    q, k, v = _qkv(52, 1, 2, 1, 10, 25, 4)
    o, l = oracle.attention_naive(q, k, v, 0.7, True, window=(0, -1))
    p = np.arange(10) + 15
    np.testing.assert_allclose(o[0, :, :, :], v[0, 0][p][None].repeat(2, 0), atol=1e-14)
    np.testing.assert_allclose(l[0], 0.7 * np.einsum("hid,id->hi", q[0], k[0, 0][p]), atol=1e-13)


def test_window_equals_attention_on_the_key_slice():
    # Every row's visible keys are one contiguous range; attention over that
    # slice alone (no mask) gives the same row.
    q, k, v = _qkv(53, 1, 2, 1, 40, 64, 8)
    for causal, win in ((True, (7, -1)), (False, (5, 3)), (False, (-1, 2)), (True, (31, 0))):
        o, l = oracle.attention_naive(q, k, v, 0.4, causal, window=win)
        for i in range(40):
            p = i + 24
            lo = 0 if win[0] < 0 else max(0, p - win[0])
            hi = p if causal else (63 if win[1] < 0 else min(63, p + win[1]))
            o1, l1 = oracle.attention_naive(q[:, :, i:i + 1], k[:, :, lo:hi + 1], v[:, :, lo:hi + 1], 0.4, False)
            np.testing.assert_allclose(o[:, :, i], o1[:, :, 0], atol=1e-13)
            np.testing.assert_allclose(l[:, :, i], l1[:, :, 0], atol=1e-13)


def test_window_lse_grows_with_the_window_and_detects_off_by_one():
    q, k, v = _qkv(54, 1, 2, 2, 20, 20, 8)
    prev = None
    for left in (0, 1, 2, 5, 19):
        _, l = oracle.attention_naive(q, k, v, 0.5, True, window=(left, -1))
        if prev is not None:
            assert np.all(l >= prev - 1e-12)
        prev = l
    # planted mistake: a window one key wider differs (rows with p >= left + 1)
    o3, _ = oracle.attention_naive(q, k, v, 0.5, True, window=(3, -1))
    o4, _ = oracle.attention_naive(q, k, v, 0.5, True, window=(4, -1))
    assert np.abs(o3 - o4)[:, :, 4:].min(axis=-1).max() > 1e-6


# ---- block-sparse mask ----

def _elementwise_mask(bm_bh, Nq, Nk, block, causal):
    """Boolean [Nq, Nk] written out entry by entry from the block mask."""
    vis = np.zeros((Nq, Nk), dtype=bool)
    for i in range(Nq):
        for j in range(Nk):
            vis[i, j] = bool(bm_bh[i // block][j // block]) and (not causal or j <= i + Nk - Nq)
    return vis


def test_block_mask_matches_sdpa_with_an_explicit_mask():
    # Library pin: torch SDPA (float64) with the element mask spelled out per
    # (query, key) from the block mask, K/V heads repeated for GQA. Every row
    # keeps at least one key (SDPA has no convention for empty rows).
    B, Hq, Hkv, Nq, Nk, d, blk = 2, 4, 2, 11, 14, 8, 3
    q, k, v = _qkv(61, B, Hq, Hkv, Nq, Nk, d)
    r = np.random.default_rng(62)
    nqb, nkb = -(-Nq // blk), -(-Nk // blk)
    for causal in (False, True):
        bm = (r.random((B, Hq, nqb, nkb)) < 0.5).astype(np.uint8)
        bm[..., -1] = 1   # the last key block: visible to every row causally too
        bm[..., 0] = 1
        o, l = oracle.attention_naive(q, k, v, 0.35, causal, block_mask=bm, block=blk)
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                vis = _elementwise_mask(bm[b, h], Nq, Nk, blk, causal)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[b, h][None]), torch.from_numpy(k[b, h // G][None]),
                    torch.from_numpy(v[b, h // G][None]), attn_mask=torch.from_numpy(vis)[None],
                    scale=0.35).numpy()[0]
                np.testing.assert_allclose(o[b, h], ref, atol=1e-12)
                s = 0.35 * q[b, h] @ k[b, h // G].T
                lse = scipy.special.logsumexp(np.where(vis, s, -np.inf), axis=1)
                np.testing.assert_allclose(l[b, h], lse, atol=1e-12)


def test_block_mask_all_ones_is_plain_attention_and_broadcasts():
    q, k, v = _qkv(63, 2, 4, 1, 300, 260, 8)
    for causal in (False, True):
        o, l = oracle.attention_naive(q, k, v, 0.2, causal)
        o2, l2 = oracle.attention_naive(q, k, v, 0.2, causal, block_mask=np.ones((1, 1, 3, 3), np.uint8))
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(l, l2)


def test_block_diagonal_mask_is_independent_attention_per_block():
    # Only the diagonal block pairs set (Nq == Nk): each 128-query block
    # attends to its own 128 keys, i.e. separate attention problems.
    q, k, v = _qkv(64, 1, 2, 2, 300, 300, 8)
    bm = np.eye(3, dtype=np.uint8)[None, None]
    for causal in (False, True):
        o, l = oracle.attention_naive(q, k, v, 0.5, causal, block_mask=bm)
        for c in range(3):
            sl = slice(128 * c, min(300, 128 * (c + 1)))
            o1, l1 = oracle.attention_naive(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.5, causal)
            np.testing.assert_allclose(o[:, :, sl], o1, atol=1e-13)
            np.testing.assert_allclose(l[:, :, sl], l1, atol=1e-13)


def test_single_key_block_is_attention_on_that_slice_and_empty_rows():
    q, k, v = _qkv(65, 1, 2, 1, 200, 400, 4)
    bm = np.zeros((1, 1, 2, 4), np.uint8)
    bm[0, 0, 0, 2] = 1   # query block 0 sees keys 256..383 only; query block 1 nothing
    o, l = oracle.attention_naive(q, k, v, 0.6, False, block_mask=bm)
    o1, l1 = oracle.attention_naive(q[:, :, :128], k[:, :, 256:384], v[:, :, 256:384], 0.6, False)
    np.testing.assert_allclose(o[:, :, :128], o1, atol=1e-13)
    np.testing.assert_allclose(l[:, :, :128], l1, atol=1e-13)
    assert np.all(o[:, :, 128:] == 0) and np.all(np.isneginf(l[:, :, 128:]))


def test_block_mask_per_head():
    # Each query head uses its own mask: head h alone under mask[h] gives the same rows.
    q, k, v = _qkv(66, 1, 4, 2, 140, 270, 8)
    r = np.random.default_rng(67)
    bm = (r.random((1, 4, 2, 3)) < 0.6).astype(np.uint8)
    bm[..., 0] = 1
    o, l = oracle.attention_naive(q, k, v, 0.3, True, block_mask=bm)
    for h in range(4):
        o1, l1 = oracle.attention_naive(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], 0.3, True,
                                        block_mask=bm[:, h:h + 1])
        np.testing.assert_array_equal(o[:, h], o1[:, 0])
        np.testing.assert_array_equal(l[:, h], l1[:, 0])


@pytest.mark.parametrize("kind", ["transposed", "kv_head_index", "block_edge"])
def test_block_mask_planted_mistakes_are_caught(kind, monkeypatch):
    # A copy of the oracle with the block index computed wrongly must differ
    # from the SDPA pin's element mask.
    B, Hq, Hkv, Nq, Nk, d, blk = 1, 4, 2, 9, 9, 4, 3
    q, k, v = _qkv(68, B, Hq, Hkv, Nq, Nk, d)
    r = np.random.default_rng(69)
    bm = (r.random((B, Hq, 3, 3)) < 0.5).astype(np.uint8)
    bm[..., 0] = 1
    orig = oracle._block_visible

    def mutant(mask_bh, i_rows, n_k, block):
        if kind == "transposed":
            return orig(np.ascontiguousarray(mask_bh.T), i_rows, n_k, block)
        if kind == "block_edge":
            qb = ((i_rows + 1) // block)[:, None].clip(0, mask_bh.shape[0] - 1)
            return mask_bh[qb, (np.arange(n_k) // block)[None, :]] != 0
        return orig(mask_bh, i_rows, n_k, block)

    if kind == "kv_head_index":
        bm_used = bm[:, [0, 0, 1, 1]]   # mask looked up by K/V head instead of query head
    else:
        bm_used = bm
        monkeypatch.setattr(oracle, "_block_visible", mutant)
    o, _ = oracle.attention_naive(q, k, v, 0.5, False, block_mask=bm_used, block=blk)
    monkeypatch.undo()
    worst = 0.0
    for h in range(Hq):
        vis = _elementwise_mask(bm[0, h], Nq, Nk, blk, False)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, h][None]), torch.from_numpy(k[0, h // 2][None]),
            torch.from_numpy(v[0, h // 2][None]), attn_mask=torch.from_numpy(vis)[None], scale=0.5).numpy()[0]
        worst = max(worst, np.abs(o[0, h] - ref).max())
    assert worst > 1e-6, kind


# ---- backward ----

def _autograd_grads(q, k, v, do, scale, causal, mask_fn=None):
    """torch autograd through SDPA in float64, K/V heads repeated for GQA."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    kr = kt.repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    mask = (j <= i + Nk - Nq) if causal else torch.ones(Nq, Nk, dtype=torch.bool)
    if mask_fn is not None:
        mask = mask & mask_fn(i, j)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, attn_mask=mask, scale=scale)
    o.backward(torch.from_numpy(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


BWD_SHAPES = [  # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 5, 5, 4, False), (1, 2, 1, 7, 7, 8, True), (2, 4, 2, 6, 9, 8, True),
    (1, 4, 1, 9, 4, 4, False), (1, 6, 2, 12, 12, 16, True), (1, 2, 2, 3, 11, 8, True),
]


@pytest.mark.parametrize("shape", BWD_SHAPES)
def test_backward_matches_torch_autograd(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = rnd(B, Hq, Nq, d), rnd(B, Hkv, Nk, d), rnd(B, Hkv, Nk, d)
    do = rnd(B, Hq, Nq, d)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.37, causal)
    rq, rk, rv = _autograd_grads(q, k, v, do, 0.37, causal)
    np.testing.assert_allclose(dq, rq, atol=1e-12)
    np.testing.assert_allclose(dk, rk, atol=1e-12)
    np.testing.assert_allclose(dv, rv, atol=1e-12)


def test_backward_with_window_and_block_mask_matches_autograd():
    q, k, v, do = rnd(1, 4, 10, 8), rnd(1, 2, 13, 8), rnd(1, 2, 13, 8), rnd(1, 4, 10, 8)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, True, window=(4, -1))
    rq, rk, rv = _autograd_grads(q, k, v, do, 0.5, True, mask_fn=lambda i, j: j >= i + 3 - 4)
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, atol=1e-12)
    bm = np.array([[1, 0, 1, 1], [0, 1, 1, 0], [1, 1, 0, 1]], np.uint8)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, False, block_mask=bm, block=4)
    rq, rk, rv = _autograd_grads(q, k, v, do, 0.5, False,
                                 mask_fn=lambda i, j: torch.from_numpy(bm.astype(bool))[i // 4, j // 4])
    for a, r in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(a, r, atol=1e-12)


def test_backward_matches_finite_differences():
    # Brute force: L = sum(dO * O); central differences of every input entry.
    q, k, v, do = rnd(1, 2, 4, 3), rnd(1, 1, 5, 3), rnd(1, 1, 5, 3), rnd(1, 2, 4, 3)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.8, True)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_naive(q_, k_, v_, 0.8, True)
        return float((o * do).sum())

    eps = 1e-6
    for x, gx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - gx[idx]) < 1e-7, (which, idx, fd, gx[idx])


def test_backward_single_key_closed_form():
    # Nk = 1, no mask: every P is 1, so dV = sum of dO over the group's rows
    # and heads, and dQ = dK = 0.
    q, k, v, do = rnd(1, 4, 6, 8), rnd(1, 2, 1, 8), rnd(1, 2, 1, 8), rnd(1, 4, 6, 8)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.3, False)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    np.testing.assert_allclose(dv[0, 0, 0], do[0, 0:2].sum(axis=(0, 1)), atol=1e-12)
    np.testing.assert_allclose(dv[0, 1, 0], do[0, 2:4].sum(axis=(0, 1)), atol=1e-12)


def test_backward_is_invariant_to_shifting_all_keys():
    # Adding one vector c to every key adds scale*q.c to a whole score row,
    # which the softmax removes; dS rows sum to 0, so dQ = scale dS (K + c)
    # is unchanged too.
    q, k, v, do = rnd(1, 2, 8, 8), rnd(1, 1, 8, 8), rnd(1, 1, 8, 8), rnd(1, 2, 8, 8)
    c = np.random.default_rng(9).standard_normal(8)
    a = oracle.attention_backward(q, k, v, do, 0.4, True)
    b = oracle.attention_backward(q, k + c, v, do, 0.4, True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-11)


@pytest.mark.parametrize("kind", ["no_row_term", "dq_unscaled", "dk_first_head_only", "dv_from_dp"])
def test_backward_planted_mistakes_are_caught(kind, monkeypatch):
    q, k, v, do = rnd(1, 4, 7, 8), rnd(1, 2, 7, 8), rnd(1, 2, 7, 8), rnd(1, 4, 7, 8)
    rq, rk, rv = _autograd_grads(q, k, v, do, 0.6, True)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.6, True)
    if kind == "no_row_term":      # dS = P * dP
        P = oracle.attention_naive(q, k, v, 0.6, True, return_p=True)[2]
        kr = np.repeat(k, 2, axis=1)
        vr = np.repeat(v, 2, axis=1)
        dS = P * (do @ np.swapaxes(vr, -1, -2))
        dq = 0.6 * dS @ kr
    elif kind == "dq_unscaled":
        dq = dq / 0.6
    elif kind == "dk_first_head_only":
        dk = dk.copy()
        P = oracle.attention_naive(q, k, v, 0.6, True, return_p=True)[2]
        vr = np.repeat(v, 2, axis=1)
        dP = do @ np.swapaxes(vr, -1, -2)
        dS = P * (dP - (dP * P).sum(-1, keepdims=True))
        dk[0, 0] = 0.6 * dS[0, 0].T @ q[0, 0]
        dk[0, 1] = 0.6 * dS[0, 2].T @ q[0, 2]
    elif kind == "dv_from_dp":     # dV = dS^T dO instead of P^T dO
        P = oracle.attention_naive(q, k, v, 0.6, True, return_p=True)[2]
        vr = np.repeat(v, 2, axis=1)
        dP = do @ np.swapaxes(vr, -1, -2)
        dS = P * (dP - (dP * P).sum(-1, keepdims=True))
        dvh = np.swapaxes(dS, -1, -2) @ do
        dv = dvh[:, 0::2] + dvh[:, 1::2]
    worst = max(np.abs(dq - rq).max(), np.abs(dk - rk).max(), np.abs(dv - rv).max())
    assert worst > 1e-6, kind


# ---- FP8 (E4M3) block quantization ----

def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_e4m3_encode_matches_torch_cast():
    # Library pin: torch's float32 -> float8_e4m3fn cast (round to nearest
    # even) on random magnitudes over the whole range, every code value, every
    # midpoint between neighbouring codes (ties) and subnormals.
    r = np.random.default_rng(70)
    vals = [r.standard_normal(20000) * np.exp2(r.uniform(-12, 8.7, 20000))]
    finite = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = np.unique(finite[np.isfinite(finite)])
    vals.append(finite)
    vals.append((finite[1:] + finite[:-1]) / 2)          # ties
    vals.append(-(finite[1:] + finite[:-1]) / 2)
    x = np.concatenate(vals).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    # torch keeps the sign of a zero result; compare values for zeros, codes otherwise
    nz = oracle.e4m3_decode(ref) != 0
    np.testing.assert_array_equal(got[nz], ref[nz])
    assert np.all(oracle.e4m3_decode(got[~nz]) == 0)


def test_quantize_fp8_block_properties():
    x = np.random.default_rng(71).standard_normal((2, 3, 300, 16)).astype(np.float32)
    x[1, 2, 128:256] = 0.0                                   # an all-zero block
    codes, scales = oracle.quantize_fp8(x, 128)
    assert scales.shape == (2, 3, 3) and scales.dtype == np.float32
    assert scales[1, 2, 1] == 1.0 and np.all(codes[1, 2, 128:256] == 0)
    for b in range(2):
        for h in range(3):
            for i in range(3):
                blk = x[b, h, 128 * i:128 * (i + 1)]
                if not np.any(blk):
                    continue
                assert scales[b, h, i] == np.float32(np.abs(blk).max()) / np.float32(448)
                # the block's largest magnitude lands on the largest code, 448
                c = codes[b, h, 128 * i:128 * (i + 1)].reshape(-1)
                assert np.max(oracle.e4m3_decode(c & 0x7F)) == 448.0
    # round trip within half a code step: 2^-4 relative for normals, 2^-10 * scale for subnormals
    deq = oracle.dequantize_fp8(codes, scales, 128)
    s = np.repeat(scales, 128, axis=2)[:, :, :300, None].astype(np.float64)
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) * (1 + 1e-6))


def test_attention_fp8_is_attention_of_the_dequantized_inputs():
    # With block scales chosen as powers of two and codes given, the
    # dequantized values are exact: attention_fp8 equals attention_naive of
    # code value * scale; a wrong block (planted: all rows on block 0's
    # scale) differs.
    r = np.random.default_rng(72)
    qc = r.integers(0, 256, (1, 2, 200, 16)).astype(np.uint8) & 0xF7  # no NaN codes (S.1111.111)
    kc = r.integers(0, 256, (1, 1, 300, 16)).astype(np.uint8) & 0xF7
    vc = r.integers(0, 256, (1, 1, 300, 16)).astype(np.uint8) & 0xF7
    qs = np.exp2(r.integers(-9, -5, (1, 2, 2))).astype(np.float32)
    ks = np.exp2(r.integers(-9, -5, (1, 1, 3))).astype(np.float32)
    vs = np.array([[[2.0 ** -7]]], np.float32)
    o, l = oracle.attention_fp8(qc, qs, kc, ks, vc, vs, 0.25, True)
    q = oracle.e4m3_decode(qc) * np.repeat(qs, 128, axis=2)[:, :, :200, None]
    k = oracle.e4m3_decode(kc) * np.repeat(ks, 128, axis=2)[:, :, :300, None]
    v = oracle.e4m3_decode(vc) * 2.0 ** -7
    o2, l2 = oracle.attention_naive(q, k, v, 0.25, True)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(l, l2, atol=1e-12)
    k_wrong = oracle.e4m3_decode(kc) * ks[:, :, :1, None]
    o3, _ = oracle.attention_naive(q, k_wrong, v, 0.25, True)
    assert np.abs(o3 - o).max() > 1e-6
