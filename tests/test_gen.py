"""The seeded input generator: pinned to SplitMix64's and Box-Muller's published
definitions (re-derived here in plain Python), plus the properties the tests
and the bench rely on (determinism, independence of streams, layout rules)."""
import math
import struct

import numpy as np
import pytest
import torch

import gen

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def py_splitmix_next(state):
    """One step of SplitMix64 as published: advance by gamma, then mix."""
    state = (state + GAMMA) & M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return state, z ^ (z >> 31)


def py_nth_output(seed, n):
    """n-th output (0-based) of a SplitMix64 generator seeded with `seed`."""
    st = seed & M64
    out = None
    for _ in range(n + 1):
        st, out = py_splitmix_next(st)
    return out


def test_draw_matches_published_splitmix64():
    for seed, stream, idx in [(0, 0, 0), (1003, 1, 5), (2**63 + 7, 4, 17), (42, 5, 0)]:
        key = py_nth_output(seed, stream)
        assert gen.draw(seed, stream, idx) == py_nth_output(key, idx)


def test_splitmix64_known_vector():
    # Seed 1234567: the generator's first outputs as printed in Vigna's public
    # reference implementation's test vector.
    st = 1234567
    outs = []
    for _ in range(3):
        st, o = py_splitmix_next(st)
        outs.append(o)
    assert outs == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def py_normal(seed, stream, e):
    key = py_nth_output(seed, stream)
    p = e // 2
    u1 = ((py_nth_output(key, 2 * p) >> 11) + 1) * 2.0 ** -53
    u2 = ((py_nth_output(key, 2 * p + 1) >> 11) + 1) * 2.0 ** -53
    r = math.sqrt(-2.0 * math.log(u1))
    t = 2.0 * math.pi * u2
    return r * (math.sin(t) if e & 1 else math.cos(t))


def test_normals_match_box_muller():
    seed, stream = 1002, 2
    got = gen.normal_f32(seed, stream, (9,), offset=3)
    for i in range(9):
        want = struct.unpack("f", struct.pack("f", py_normal(seed, stream, 3 + i)))[0]
        assert got[i] == np.float32(want)


def test_bf16_is_round_to_nearest_even_of_the_float():
    f = gen.normal_f32(7, 0, (4096,), sigma=0.5)
    b = gen.normal_bf16(7, 0, (4096,), sigma=0.5)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_determinism_offsets_and_streams():
    a = gen.normal_bf16(5, 1, (1000,))
    assert np.array_equal(a, gen.normal_bf16(5, 1, (1000,)))
    assert np.array_equal(a[300:], gen.normal_bf16(5, 1, (700,), offset=300))
    assert not np.array_equal(a, gen.normal_bf16(5, 2, (1000,)))
    assert not np.array_equal(a, gen.normal_bf16(6, 1, (1000,)))


def test_moments():
    x = gen.normal_f32(11, 0, (1 << 20,), sigma=0.5).astype(np.float64)
    assert abs(x.mean()) < 3 * 0.5 / 1024
    assert abs(x.std() - 0.5) < 0.005


def test_uniform_int_range_and_permutation():
    u = gen.uniform_int(3, 3, 10000, 512, 32768)
    assert u.min() >= 512 and u.max() <= 32768
    p = gen.permutation(3, 4, 1000)
    assert np.array_equal(np.sort(p), np.arange(1000))
    assert not np.array_equal(p, np.arange(1000))


def test_decode_layout_rules():
    lens, table, total = gen.decode_layout(1004, 64, 512, 32768, 16, 2048)
    assert lens.dtype == np.int32 and table.dtype == np.int32 and table.shape == (64, 2048)
    npages = (lens.astype(np.int64) + 15) // 16
    assert total == int(npages.sum())
    used = np.concatenate([table[b, :npages[b]] for b in range(64)])
    assert np.array_equal(np.sort(used), np.arange(total))       # a bijection onto the pool
    for b in range(64):
        assert (table[b, npages[b]:] == -1).all()                 # unused entries are -1


def test_row_sample():
    r = gen.row_sample(1004, 65536, 256, salt=3)
    assert r.size == 256 and r[0] == 0 and r[-1] == 65535
    assert np.unique(r).size == 256
    assert not np.array_equal(r, gen.row_sample(1004, 65536, 256, salt=4))


def test_random_block_mask_is_seeded_and_has_its_density():
    a = gen.random_block_mask(7, (2, 3, 40, 50), 30)
    b = gen.random_block_mask(7, (2, 3, 40, 50), 30)
    assert a.dtype == np.uint8 and a.shape == (2, 3, 40, 50)
    np.testing.assert_array_equal(a, b)
    assert set(np.unique(a)) <= {0, 1}
    assert abs(a.mean() - 0.30) < 0.03
    # entry e is draw e of stream 6 compared with the percentage
    u = gen.uniform_int(7, gen.STREAM_MASK, 12000, 0, 99)
    np.testing.assert_array_equal(a.reshape(-1), (u < 30).astype(np.uint8))
    assert gen.random_block_mask(7, (5,), 0).sum() == 0 and gen.random_block_mask(7, (5,), 100).sum() == 5


def test_local_global_block_mask():
    m = gen.local_global_block_mask(6, 6, 2, 1)
    expect = np.array([[1, 0, 0, 0, 0, 0],
                       [1, 1, 0, 0, 0, 0],
                       [1, 1, 1, 0, 0, 0],
                       [1, 0, 1, 1, 0, 0],
                       [1, 0, 0, 1, 1, 0],
                       [1, 0, 0, 0, 1, 1]], dtype=np.uint8)
    np.testing.assert_array_equal(m, expect)


def test_outlier_bf16_enlarges_the_drawn_entries_exactly():
    shape = (2, 3, 1000, 16)
    base = gen.normal_bf16(9, gen.STREAM_K, shape)
    out = gen.outlier_bf16(9, gen.STREAM_K, shape)
    pick = gen.uniform_int(9, gen.STREAM_OUTLIER, base.size, 0, 999999, offset=gen.STREAM_K << 40) < 1000
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).reshape(-1)
    np.testing.assert_array_equal(f(out)[pick], f(base)[pick] * 16)
    np.testing.assert_array_equal(out.reshape(-1)[~pick], base.reshape(-1)[~pick])
    assert abs(pick.mean() - 1e-3) < 3e-4
    # Q and K draw their outlier positions from different sub-sequences
    assert not np.array_equal(pick, gen.uniform_int(9, gen.STREAM_OUTLIER, base.size, 0, 999999,
                                                    offset=gen.STREAM_Q << 40) < 1000)
    with pytest.raises(ValueError):
        gen.outlier_bf16(9, gen.STREAM_K, shape, factor=10.0)


def test_random_signs():
    s = gen.random_signs(5, 4096)
    assert s.dtype == np.int8 and set(np.unique(s).tolist()) == {-1, 1}
    assert abs(float(s.mean())) < 0.06
    np.testing.assert_array_equal(s, 1 - 2 * gen.uniform_int(5, gen.STREAM_SIGNS, 4096, 0, 1))
