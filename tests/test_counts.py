"""CPU pins of the closed-form visible-key counts that the GPU exact tests
(test_gpu_exact.py) compare rint(exp(LSE)) against: with Q = 0 the oracle's
LSE is ln(count), so both must agree on every row, and a one-key shift of
either window edge or of a block edge must not."""
import numpy as np
import pytest

import gen
import oracle
from test_gpu_exact import block_counts, window_counts


def _oracle_counts(Nq, Nk, causal, window=None, block_mask=None):
    q = np.zeros((1, 1, Nq, 4))
    kv = np.ones((1, 1, Nk, 4))
    _, l = oracle.attention_naive(q, kv, kv, 0.5, causal, window=window, block_mask=block_mask)
    l = l[0, 0]
    fin = np.isfinite(l)
    return np.where(fin, np.rint(np.exp(np.where(fin, l, 0.0))), 0).astype(np.int64)


@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (300, 300, True, (100, -1)), (90, 200, True, (51, -1)), (100, 100, False, (10, 7)),
    (100, 100, False, (-1, 3)), (50, 60, True, None), (60, 50, True, None), (40, 40, True, (0, -1)),
    (70, 30, False, (5, 5)),
])
def test_window_counts_match_oracle(Nq, Nk, causal, window):
    want = _oracle_counts(Nq, Nk, causal, window=window)
    assert np.array_equal(window_counts(Nq, Nk, causal, window), want)
    if window is not None and window[0] > 0:   # a left edge one key wider is caught
        assert not np.array_equal(window_counts(Nq, Nk, causal, (window[0] + 1, window[1])), want)


@pytest.mark.parametrize("Nq,Nk,causal", [(300, 300, True), (200, 500, False), (500, 200, True), (129, 257, True)])
def test_block_counts_match_oracle(Nq, Nk, causal):
    m = gen.random_block_mask(5 + Nq, (1, 1, -(-Nq // 128), -(-Nk // 128)), 50)
    want = _oracle_counts(Nq, Nk, causal, block_mask=m)
    assert np.array_equal(block_counts(m[0, 0], Nq, Nk, causal), want)
    assert not np.array_equal(block_counts(m[0, 0], Nq, Nk, causal, block=127), want)
