"""The FP8 forward's O bar must bind (CPU only, no GPU).

A model of the FP8 kernel's arithmetic runs on the CPU: scores in exp2
units against a lazily moved reference (it moves only when a 128-key tile's
maximum exceeds it by more than 8), each tile's probabilities rounded to E4M3
(oracle.e4m3_encode / e4m3_decode) before the P.V product, the row sum taken
from the unrounded probabilities, and O rounded to bf16. That model must pass
the bar of fa_cases.fp8_bound_terms / fp8_bars on the timed FP8 workload's
shape (causal GQA 64/8, N = 8192, d = 128, one K/V head group, 64 sampled rows
per head), and plausible kernel mistakes must fail it: an O of zeros, key
tile 1 multiplied with key tile 0's values, every tile's probabilities paired
with the previous tile's values (a wrong LDS stage), every tile's values
weighted by the previous tile's probabilities. The FP8 format itself
("FlashAttention" glossary page, section "FlashAttention-3": FP8 with block
quantization) is pinned in test_oracle.py.
"""
import math

import numpy as np
import pytest

import gen
import oracle
from fa_cases import f64_to_bf16_bits, fp8_bars, fp8_bound_terms

TILE = 128
SLACK = 8.0


def model_fp8_kernel(qd, kd, vd, scale, causal, rows, mistake=None):
    """O of the FP8 kernel's arithmetic for the sampled rows [1, Hq, R]."""
    B, Hq, Nq, d = qd.shape
    Hkv, Nk = kd.shape[1], kd.shape[2]
    G = Hq // Hkv
    R = rows.shape[-1]
    out = np.zeros((B, Hq, R, d))
    c = scale * math.log2(math.e)
    for h in range(Hq):
        g = h // G
        ii = rows[0, h]
        S = (qd[0, h, ii] @ kd[0, g].T) * c
        if causal:
            S = np.where(np.arange(Nk)[None, :] <= ii[:, None] + (Nk - Nq), S, -np.inf)
        ref = np.full(R, -np.inf)
        l = np.zeros(R)
        acc = np.zeros((R, d))
        p_prev = None
        for j0 in range(0, Nk, TILE):
            St = S[:, j0:j0 + TILE]
            tmax = St.max(axis=1)
            new = np.where(tmax > ref + SLACK, np.maximum(ref, tmax), ref)
            fin_old, fin_new = np.isfinite(ref), np.isfinite(new)
            alpha = np.where(fin_old, np.exp2(np.where(fin_old, ref, 0.0) - np.where(fin_new, new, 0.0)), 1.0)
            acc *= alpha[:, None]
            l *= alpha
            ref = new
            pt = np.where(np.isfinite(St), np.exp2(St - np.where(np.isfinite(ref), ref, 0.0)[:, None]), 0.0)
            pq = oracle.e4m3_decode(oracle.e4m3_encode(pt))
            l += pt.sum(axis=1)
            vt = vd[0, g, j0:j0 + TILE]
            if mistake == "tile1_uses_tile0_v" and j0 == TILE:
                vt = vd[0, g, 0:TILE]
            if mistake == "v_from_previous_stage" and j0 >= TILE:
                vt = vd[0, g, j0 - TILE:j0 - TILE + pt.shape[1]]
            if mistake == "p_from_previous_tile":
                cur = pq
                pq = np.zeros_like(pq) if p_prev is None else p_prev[:, :pq.shape[1]]
                p_prev = cur
            acc += pq @ vt
        o = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        out[0, h] = oracle.bf16_bits_to_f64(f64_to_bf16_bits(o))
    return out


def _c3_group(kv_head=3, n_rows=64, transform=None):
    """K/V head `kv_head` of the causal GQA 64/8 N=8192 d=128 inputs (seed
    1003) and its 8 query heads, quantized like the timed FP8 workload."""
    N, d = 8192, 128
    f = oracle.bf16_bits_to_f64
    q = f(gen.normal_bf16(1003, gen.STREAM_Q, (1, 64, N, d)))[:, 8 * kv_head:8 * kv_head + 8]
    k = f(gen.normal_bf16(1003, gen.STREAM_K, (1, 8, N, d)))[:, kv_head:kv_head + 1]
    v = f(gen.normal_bf16(1003, gen.STREAM_V, (1, 8, N, d)))[:, kv_head:kv_head + 1]
    if transform is not None:
        q, k = transform(q, k)
    qc, qs = oracle.quantize_fp8(q, 128)
    kc, ks = oracle.quantize_fp8(k, 128)
    vc, vs = oracle.quantize_fp8(v, N)
    qd, kd, vd = oracle.dequantize_fp8(qc, qs, 128), oracle.dequantize_fp8(kc, ks, 128), oracle.dequantize_fp8(vc, vs, N)
    rows = np.stack([np.stack([gen.row_sample(1003, N, n_rows, salt=1000 + 8 * kv_head + h) for h in range(8)])])
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o_ref, _ = oracle.attention_fp8(qc, qs, kc, ks, vc, vs, scale, True, rows=rows)
    D, R, _, _ = fp8_bound_terms(qd, kd, vd, scale, True, rows=rows)
    return qd, kd, vd, rows, scale, o_ref, D, R


@pytest.fixture(scope="module")
def c3_group():
    return _c3_group()


def _ratios(got, o_ref, D, R):
    bound, mean_bar = fp8_bars(D, R, o_ref)
    err = np.abs(got - o_ref)
    return float((err / bound).max()), float(err.mean()) / mean_bar


def test_bar_binds_on_the_longest_row(c3_group):
    """At row 8191 (8192 visible keys) the element-wise bound sits below the
    row's own |O| scale (its RMS) everywhere, and below half of it for the
    median element, so it constrains the value."""
    qd, kd, vd, rows, scale, o_ref, D, R = c3_group
    bound, _ = fp8_bars(D, R, o_ref)
    last = rows[0, 0] == 8191
    assert last.any()
    rms = float(np.sqrt((o_ref[0, 0, last] ** 2).mean()))
    b = bound[0, 0, last]
    assert float(b.max()) < rms and float(np.median(b)) < 0.5 * rms, (float(b.max()), float(np.median(b)), rms)


def test_model_of_the_kernel_passes(c3_group):
    qd, kd, vd, rows, scale, o_ref, D, R = c3_group
    worst, mean_ratio = _ratios(model_fp8_kernel(qd, kd, vd, scale, True, rows), o_ref, D, R)
    assert worst <= 0.6 and mean_ratio <= 0.5, (worst, mean_ratio)


@pytest.mark.parametrize("mistake", ["zeros", "tile1_uses_tile0_v", "v_from_previous_stage",
                                     "p_from_previous_tile"])
def test_planted_mistakes_fail(mistake, c3_group):
    qd, kd, vd, rows, scale, o_ref, D, R = c3_group
    got = np.zeros_like(o_ref) if mistake == "zeros" else \
        model_fp8_kernel(qd, kd, vd, scale, True, rows, mistake=mistake)
    worst, mean_ratio = _ratios(got, o_ref, D, R)
    # each mistake must fail both the element-wise and the mean bar
    assert worst > 1.0 and mean_ratio > 1.0, (mistake, worst, mean_ratio)


def test_model_passes_on_rising_scores():
    """Keys scaled by a ramp: the row maximum keeps rising, the reference
    moves on later tiles and rows turn peaky (many subnormal and flushed
    probabilities)."""
    def ramp(q, k):
        n = k.shape[-2]
        return q, k * (0.5 + 3.5 * np.arange(n) / (n - 1))[:, None]
    qd, kd, vd, rows, scale, o_ref, D, R = _c3_group(kv_head=1, n_rows=32, transform=ramp)
    worst, mean_ratio = _ratios(model_fp8_kernel(qd, kd, vd, scale, True, rows), o_ref, D, R)
    assert worst <= 1.0 and mean_ratio <= 1.0, (worst, mean_ratio)
