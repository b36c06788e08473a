"""Shared helpers for the GPU parity tests: seeded inputs (from gen), expected
values (from oracle, on the CPU, in float64) and the comparison bar.

Tolerance (float outputs, from the project's acceptance bar): O max-abs
<= 1e-2 and mean-abs <= 1e-3; LSE |diff| <= 1e-3 * max(1, |LSE_ref|).
Why it is enough and not loose: O is a convex combination of bf16 values of
size O(1) rounded once to bf16 (half-ulp 2^-9 * |O| ~ 4e-3 at |O| ~ 2), and
the kernel's only other rounding is P to bf16 (relative 2^-9 per weight,
averaging out over the row) and fp32 accumulation.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import gen
import oracle

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_REL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


class PrefillCase:
    def __init__(self, B, Hq, Hkv, Nq, Nk, d, causal, seed, sigma=1.0, scale=None, window=None, block_mask=None):
        self.B, self.Hq, self.Hkv, self.Nq, self.Nk, self.d = B, Hq, Hkv, Nq, Nk, d
        self.causal = causal
        self.window = window  # None, or (left, right) for fa_forward_window
        # None, or a uint8 [B or 1, Hq or 1, ceil(Nq/128), ceil(Nk/128)] mask for fa_forward_block_sparse
        self.block_mask = block_mask
        self.seed = seed
        self.sigma = sigma
        self.scale = float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale))
        self.q_bits = gen.normal_bf16(seed, gen.STREAM_Q, (B, Hq, Nq, d), sigma)
        self.k_bits = gen.normal_bf16(seed, gen.STREAM_K, (B, Hkv, Nk, d), sigma)
        self.v_bits = gen.normal_bf16(seed, gen.STREAM_V, (B, Hkv, Nk, d), sigma)

    def run_gpu(self, q_bits=None, k_bits=None, v_bits=None):
        import exact_attention_03_amd as fa
        q = to_dev_bf16(self.q_bits if q_bits is None else q_bits)
        k = to_dev_bf16(self.k_bits if k_bits is None else k_bits)
        v = to_dev_bf16(self.v_bits if v_bits is None else v_bits)
        o = torch.full((self.B, self.Hq, self.Nq, self.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((self.B, self.Hq, self.Nq), float("nan"), dtype=torch.float32, device="cuda")
        if self.block_mask is not None:
            m = torch.from_numpy(np.ascontiguousarray(self.block_mask)).cuda()
            fa.fa_forward_block_sparse(q, k, v, o, lse, self.causal, m, self.scale)
        elif self.window is None:
            fa.fa_forward(q, k, v, o, lse, self.causal, self.scale)
        else:
            fa.fa_forward_window(q, k, v, o, lse, self.causal, self.window[0], self.window[1], self.scale)
        torch.cuda.synchronize()
        return o, lse

    def oracle(self, rows=None, q_bits=None, k_bits=None, v_bits=None):
        q = oracle.bf16_bits_to_f64(self.q_bits if q_bits is None else q_bits)
        k = oracle.bf16_bits_to_f64(self.k_bits if k_bits is None else k_bits)
        v = oracle.bf16_bits_to_f64(self.v_bits if v_bits is None else v_bits)
        return oracle.attention_naive(q, k, v, self.scale, self.causal, rows=rows, window=self.window,
                                      block_mask=self.block_mask)


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, what="",
            v_absmax: float | None = None, mean_bar: float | None = None):
    """Assert the acceptance bar; returns (max_abs, mean_abs, lse_err).

    With v_absmax given (inputs far from unit variance), O is held instead to
    the element-wise bound of its bf16 arithmetic: P rounded to bf16 moves O
    by at most 2^-9 * max|V|, and the bf16 output by at most 2^-9 * |O|; the
    check allows twice their sum. mean_bar (required with v_absmax) is the
    mean-abs bar of that arithmetic (bf16_mean_bar)."""
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape
    fin = np.isfinite(lse_ref)
    # rows with no visible key: exactly O = 0 and LSE = -inf
    assert np.array_equal(np.isneginf(lse_gpu), ~fin), what + ": -inf LSE rows differ"
    assert (o_gpu[~fin] == 0).all(), what + ": rows without visible keys must be 0"
    assert np.isfinite(o_gpu).all(), what + ": non-finite O"
    d = np.abs(o_gpu - o_ref)
    max_abs = float(d.max()) if d.size else 0.0
    mean_abs = float(d.mean()) if d.size else 0.0
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    lse_err = float(lerr.max()) if lerr.size else 0.0
    say("  %s: O max|d|=%.3e mean|d|=%.3e  LSE rel=%.3e" % (what, max_abs, mean_abs, lse_err))
    if v_absmax is not None:
        bound = 2.0 * 2.0 ** -9 * (v_absmax + np.abs(o_ref))
        worst = float((d / bound).max()) if d.size else 0.0
        say("  %s: worst |d| / bf16 bound = %.3f, mean|d| / bf16 mean bar = %.3f" % (what, worst, mean_abs / mean_bar))
        assert worst <= 1.0, "%s: O exceeds its bf16 arithmetic bound (%.3f)" % (what, worst)
        assert mean_abs <= mean_bar, "%s: O mean-abs %.3e above its bf16 bar %.3e" % (what, mean_abs, mean_bar)
    else:
        assert max_abs <= O_MAX_ABS, "%s: O max-abs %.3e" % (what, max_abs)
        assert mean_abs <= O_MEAN_ABS, "%s: O mean-abs %.3e" % (what, mean_abs)
    assert lse_err <= LSE_REL, "%s: LSE rel %.3e" % (what, lse_err)
    return max_abs, mean_abs, lse_err


class DecodeCase:
    def __init__(self, B, Hq, Hkv, d, seed, len_lo=512, len_hi=32768, seq_lens=None, page_size=16,
                 max_pages_per_seq=None, max_seq_len=None, sigma=1.0):
        self.B, self.Hq, self.Hkv, self.d, self.ps = B, Hq, Hkv, d, page_size
        self.seed = seed
        self.scale = float(np.float32(1.0 / math.sqrt(d)))
        if max_pages_per_seq is None:
            hi = len_hi if seq_lens is None else max(1, max(seq_lens))
            max_pages_per_seq = max(1, -(-hi // page_size))
        self.seq_lens, self.table, self.total_pages = gen.decode_layout(
            seed, B, len_lo, len_hi, page_size, max_pages_per_seq, seq_lens=seq_lens)
        self.num_pages = max(1, self.total_pages)
        self.max_seq_len = (int(self.seq_lens.max()) if B else 1) if max_seq_len is None else max_seq_len
        self.max_seq_len = max(1, self.max_seq_len)
        self.q_bits = gen.normal_bf16(seed, gen.STREAM_Q, (B, Hq, d), sigma)
        self.k_bits = gen.normal_bf16(seed, gen.STREAM_K, (self.num_pages, Hkv, page_size, d), sigma)
        self.v_bits = gen.normal_bf16(seed, gen.STREAM_V, (self.num_pages, Hkv, page_size, d), sigma)

    def run_gpu(self, q_bits=None, k_bits=None, v_bits=None, table=None):
        import exact_attention_03_amd as fa
        q = to_dev_bf16(self.q_bits if q_bits is None else q_bits)
        kp = to_dev_bf16(self.k_bits if k_bits is None else k_bits)
        vp = to_dev_bf16(self.v_bits if v_bits is None else v_bits)
        bt = torch.from_numpy(self.table if table is None else table).cuda()
        sl = torch.from_numpy(self.seq_lens).cuda()
        o = torch.full((self.B, self.Hq, self.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((self.B, self.Hq), float("nan"), dtype=torch.float32, device="cuda")
        nbytes = fa.fa_paged_decode_workspace_size(self.B, self.Hq, self.d, self.ps, self.max_seq_len)
        ws = torch.full((max(1, nbytes) // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
        fa.fa_paged_decode(q, kp, vp, bt, sl, o, lse, self.max_seq_len, self.scale, ws, page_size=self.ps)
        torch.cuda.synchronize()
        return o, lse

    def oracle(self, q_bits=None, k_bits=None, v_bits=None, table=None):
        q = self.q_bits if q_bits is None else q_bits
        kp = self.k_bits if k_bits is None else k_bits
        vp = self.v_bits if v_bits is None else v_bits
        return oracle.paged_decode(q, kp, vp, self.table if table is None else table, self.seq_lens,
                                   self.scale, self.ps)


class PagedPrefillCase:
    """A chunk of new queries per sequence against a paged cache: seq_lens[b]
    cached tokens (the chunk's own included) in seeded-permutation pages,
    q_lens[b] query rows packed [total_q, Hq, d]. window = (left, right) runs
    fa_paged_prefill_window."""

    def __init__(self, Hq, Hkv, d, seed, seq_lens, q_lens, causal=True, page_size=16, sigma=1.0, window=None):
        self.window = window
        self.B = len(seq_lens)
        self.Hq, self.Hkv, self.d, self.ps, self.causal, self.seed = Hq, Hkv, d, page_size, causal, seed
        self.scale = float(np.float32(1.0 / math.sqrt(d)))
        max_pages = max(1, -(-max(1, max(seq_lens)) // page_size))
        self.seq_lens, self.table, self.total_pages = gen.decode_layout(
            seed, self.B, 1, 1, page_size, max_pages, seq_lens=seq_lens)
        self.num_pages = max(1, self.total_pages)
        self.q_lens = np.asarray(q_lens, dtype=np.int32)
        self.cu = np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)
        self.total_q = int(self.cu[-1])
        self.max_q_len = int(self.q_lens.max()) if self.B else 0
        self.q_bits = gen.normal_bf16(seed, gen.STREAM_Q, (self.total_q, Hq, d), sigma)
        self.k_bits = gen.normal_bf16(seed, gen.STREAM_K, (self.num_pages, Hkv, page_size, d), sigma)
        self.v_bits = gen.normal_bf16(seed, gen.STREAM_V, (self.num_pages, Hkv, page_size, d), sigma)

    def run_gpu(self):
        import exact_attention_03_amd as fa
        q, kp, vp = to_dev_bf16(self.q_bits), to_dev_bf16(self.k_bits), to_dev_bf16(self.v_bits)
        bt = torch.from_numpy(self.table).cuda()
        sl = torch.from_numpy(self.seq_lens).cuda()
        cu = torch.from_numpy(self.cu).cuda()
        o = torch.full((self.total_q, self.Hq, self.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((self.total_q, self.Hq), float("nan"), dtype=torch.float32, device="cuda")
        if self.window is None:
            fa.fa_paged_prefill(q, kp, vp, bt, sl, cu, o, lse, self.max_q_len, self.causal, self.scale,
                                page_size=self.ps)
        else:
            fa.fa_paged_prefill_window(q, kp, vp, bt, sl, cu, o, lse, self.max_q_len, self.causal,
                                       self.window[0], self.window[1], self.scale, page_size=self.ps)
        torch.cuda.synchronize()
        return o, lse

    def oracle(self):
        return oracle.paged_prefill(self.q_bits, self.k_bits, self.v_bits, self.table, self.seq_lens,
                                    self.cu, self.scale, self.causal, self.ps, window=self.window)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bf16 bit patterns (via float32, round-to-nearest-even)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


class BackwardCase:
    """fa_backward against oracle.attention_backward on gen inputs (q, k, v,
    dO from streams 0, 1, 2, 7). The GPU gets O and LSE either from the
    oracle's forward (O rounded to bf16) or from fa_forward on the GPU."""

    def __init__(self, B, Hq, Hkv, Nq, Nk, d, causal, seed, window=None, block_mask=None):
        self.B, self.Hq, self.Hkv, self.Nq, self.Nk, self.d = B, Hq, Hkv, Nq, Nk, d
        self.causal, self.seed = causal, seed
        self.window = window  # None, or (left, right) for fa_forward_window / fa_backward_window
        # None, or a uint8 [B or 1, Hq or 1, ceil(Nq/128), ceil(Nk/128)] mask for the block-sparse pair
        self.block_mask = block_mask
        self.scale = float(np.float32(1.0 / math.sqrt(d)))
        self.q_bits = gen.normal_bf16(seed, gen.STREAM_Q, (B, Hq, Nq, d))
        self.k_bits = gen.normal_bf16(seed, gen.STREAM_K, (B, Hkv, Nk, d))
        self.v_bits = gen.normal_bf16(seed, gen.STREAM_V, (B, Hkv, Nk, d))
        self.do_bits = gen.normal_bf16(seed, gen.STREAM_DO, (B, Hq, Nq, d))

    def oracle(self):
        q, k, v, do = (oracle.bf16_bits_to_f64(x) for x in (self.q_bits, self.k_bits, self.v_bits, self.do_bits))
        o, lse = oracle.attention_naive(q, k, v, self.scale, self.causal, window=self.window,
                                        block_mask=self.block_mask)
        dq, dk, dv = oracle.attention_backward(q, k, v, do, self.scale, self.causal, window=self.window,
                                               block_mask=self.block_mask)
        return o, lse, dq, dk, dv

    def run_gpu(self, o_ref=None, lse_ref=None):
        import exact_attention_03_amd as fa
        q, k, v, do = (to_dev_bf16(x) for x in (self.q_bits, self.k_bits, self.v_bits, self.do_bits))
        B, Hq, Hkv, Nq, Nk, d = self.B, self.Hq, self.Hkv, self.Nq, self.Nk, self.d
        mask = None if self.block_mask is None else \
            torch.from_numpy(np.ascontiguousarray(self.block_mask)).cuda()
        if o_ref is None:  # the GPU forward's outputs
            o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
            if mask is not None:
                fa.fa_forward_block_sparse(q, k, v, o, lse, self.causal, mask, self.scale)
            elif self.window is None:
                fa.fa_forward(q, k, v, o, lse, self.causal, self.scale)
            else:
                fa.fa_forward_window(q, k, v, o, lse, self.causal, self.window[0], self.window[1], self.scale)
        else:
            o = to_dev_bf16(f64_to_bf16_bits(o_ref))
            lse = torch.from_numpy(np.asarray(lse_ref, dtype=np.float32)).cuda()
        dq = torch.full((B, Hq, Nq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        dk = torch.full((B, Hkv, Nk, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        dv = torch.full((B, Hkv, Nk, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws_bytes = fa.fa_backward_workspace_size(B, Hq, Nq) if mask is None else \
            fa.fa_backward_block_sparse_workspace_size(B, Hq, Hkv, Nq, Nk, d)
        ws = torch.full((max(1, ws_bytes) // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
        if mask is not None:
            fa.fa_backward_block_sparse(q, k, v, o, lse, do, dq, dk, dv, self.causal, mask, self.scale, ws)
        elif self.window is None:
            fa.fa_backward(q, k, v, o, lse, do, dq, dk, dv, self.causal, self.scale, ws)
        else:
            fa.fa_backward_window(q, k, v, o, lse, do, dq, dk, dv, self.causal, self.window[0], self.window[1],
                                  self.scale, ws)
        torch.cuda.synchronize()
        return bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)


# Backward bar, relative to each gradient's own scale: max |err| <=
# GRAD_MAX_REL * max |ref| and mean |err| <= GRAD_MEAN_REL * mean |ref|.
# Why: the gradients are written in bf16, whose rounding alone moves an
# element by up to 2^-8 of its magnitude (half an ulp at the bottom of a
# binade); P and dS enter the products rounded to bf16 as well (2^-8
# relative each, averaging out over a row). 2^-6 of the largest gradient is
# 4x the output rounding; the mean bar 2^-7 is ~3x the typical combined
# effect (about 2.3e-3 of the mean gradient, measured on MI355X).
GRAD_MAX_REL = 2.0 ** -6
GRAD_MEAN_REL = 2.0 ** -7


def compare_grads(got, ref, what=""):
    out = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert g.shape == r.shape
        assert np.isfinite(g).all(), "%s %s: non-finite" % (what, name)
        err = np.abs(g - r)
        mx = float(err.max()) if err.size else 0.0
        mn = float(err.mean()) if err.size else 0.0
        scale_max = float(np.abs(r).max()) if r.size else 0.0
        scale_mean = float(np.abs(r).mean()) if r.size else 0.0
        say("  %s %s: max|d|=%.3e (%.2e of max|ref| %.3e)  mean|d|=%.3e (%.2e of mean|ref|)" % (
            what, name, mx, mx / max(scale_max, 1e-30), scale_max, mn, mn / max(scale_mean, 1e-30)))
        assert mx <= GRAD_MAX_REL * scale_max + 1e-6, "%s %s max" % (what, name)
        assert mn <= GRAD_MEAN_REL * scale_mean + 1e-7, "%s %s mean" % (what, name)
        out.append((mx, mn))
    return out


# ---------------------------------------------------------------- FP8 bar
# FP8 forward: P is rounded to E4M3 before the P.V product, O is then
# rounded to bf16. The bar below follows that arithmetic key by key.
#
# In the kernel, key j of a row gets Pt_j = exp2(s_j - ref) against the
# running reference ref <= M (the row's true maximum; the reference only
# ever takes values of scores seen so far). Pt_j is rounded to E4M3 and the
# row sum l = sum_j Pt_j is accumulated unrounded; a later move of the
# reference multiplies both by the same alpha <= 1. Normalised by l, the
# rounding error of key j is e_j * alpha_j / l, where
#   * |e_j| <= Pt_j always (0 is a code, rounding is to nearest), i.e. the
#     normalised error is at most P_j (the exact probability);
#   * a normal code (Pt_j >= 2^-6, 3 mantissa bits) moves by <= 2^-4 Pt_j,
#     i.e. <= 2^-4 P_j normalised;
#   * a subnormal one (steps of 2^-9) by <= 2^-10 absolute, i.e. <= 2^-10 / l
#     <= 2^-10 / l_max normalised, where l_max = sum_j exp(S_j - M) =
#     1 / max_j P_j (the kernel's l, against ref <= M, is at least l_max).
# Keys with exp(S_j - M) < 2^-10 (set T) may be flushed to zero: their error
# is one-signed, so it is counted deterministically, D = sum_{j in T} P_j |V_j|.
# The other keys' errors are treated as independent and zero-mean -- the
# usual probabilistic model of rounding errors (Higham & Mary, "A new
# approach to probabilistic rounding error analysis", SIAM J. Sci. Comput.
# 2019) -- each bounded by b_j = max(2^-4 P_j, 2^-10 / l_max). By
# Hoeffding's inequality their sum exceeds lam * sqrt(sum_j b_j^2 V_j^2)
# with probability <= 2 exp(-lam^2 / 2): 3e-8 per element at lam = 6.
# O is then rounded to bf16 (<= 2^-8 relative). Element-wise bar:
#   |dO| <= (D + lam * R) * (1 + 2^-8) + 2^-8 |O_ref| + 1e-6,
#   R = sqrt(sum_{j not in T} b_j^2 V_j^2).
# Mean bar (over every compared element): the mean of |random part| is at
# most its RMS, R; the bf16 rounding averages at most 2^-9 |O|:
#   mean |dO| <= mean(D + R + 2^-9 |O_ref|) + 1e-6.
FP8_LAMBDA = 6.0


def fp8_bound_terms(q, k, v, scale, causal, rows=None):
    """D, R (see above) and the oracle's O, LSE for the dequantized inputs
    q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] (float64), head by head; rows as for
    oracle.attention_naive. Uses the oracle's materialised P."""
    return rounding_bound_terms(q, k, v, scale, causal, rows, rel=2.0 ** -4, sub_abs=2.0 ** -10,
                                flush=2.0 ** -10)


def rounding_bound_terms(q, k, v, scale, causal, rows=None, rel=2.0 ** -4, sub_abs=2.0 ** -10, flush=2.0 ** -10,
                         window=None, block_mask=None):
    """D and R of the rounding model above for a format whose normal values
    round within `rel` of themselves, whose subnormals within `sub_abs`, and
    whose values below `flush` times the row maximum's probability may become
    0; plus the oracle's O and LSE. Head by head, from the oracle's P."""
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    R_rows = Nq if rows is None else np.asarray(rows).shape[-1]
    D = np.zeros((B, Hq, R_rows, d))
    Rr = np.zeros((B, Hq, R_rows, d))
    O = np.zeros((B, Hq, R_rows, d))
    L = np.zeros((B, Hq, R_rows))
    for h in range(Hq):
        g = h // G
        r = None if rows is None else (np.asarray(rows) if np.asarray(rows).ndim == 1
                                       else np.asarray(rows)[:, h:h + 1])
        bm = None if block_mask is None else np.broadcast_to(block_mask, (B, Hq) + block_mask.shape[2:])[:, h:h + 1]
        o, lse, P = oracle.attention_naive(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], scale, causal,
                                           rows=r, return_p=True, window=window, block_mask=bm)
        O[:, h], L[:, h] = o[:, 0], lse[:, 0]
        P = P[:, 0]                                         # [B, R, Nk]
        pmax = P.max(axis=-1, keepdims=True) if P.shape[-1] else np.zeros(P.shape[:-1] + (1,))
        ok = pmax > 0
        tiny = P < flush * pmax                             # exp(S - M) < flush (and invisible keys)
        inv_lmax = np.where(ok, pmax, 0.0)                   # 1 / l_max
        b = np.where(tiny, 0.0, np.maximum(rel * P, sub_abs * inv_lmax))
        va = np.abs(v[:, g])                                 # [B, Nk, d]
        D[:, h] = np.where(tiny, P, 0.0) @ va
        Rr[:, h] = np.sqrt((b * b) @ (va * va))
    return D, Rr, O, L


def fp8_bars(D, R, o_ref, lam=FP8_LAMBDA):
    """Element-wise bound and the mean-abs bar (see above)."""
    elem = (D + lam * R) * (1.0 + 2.0 ** -8) + 2.0 ** -8 * np.abs(o_ref) + 1e-6
    mean = float((D + R + 2.0 ** -9 * np.abs(o_ref)).mean()) + 1e-6 if D.size else 1e-6
    return elem, mean


def bf16_mean_bar(case, rows=None):
    """Mean-abs bar of the bf16 kernel's arithmetic for a PrefillCase: P is
    rounded to bf16 (round to nearest even, <= 2^-8 relative; float32's
    exponent range, so only values below 2^-126 of the row maximum's
    probability flush), O to bf16. By the model above (no subnormal term):
    mean |dO| <= mean(D + R + 2^-9 |O_ref|) + 1e-6, R = sqrt(sum_j (2^-8 P_j)^2 V_j^2)."""
    f = oracle.bf16_bits_to_f64
    D, R, o_ref, _ = rounding_bound_terms(f(case.q_bits), f(case.k_bits), f(case.v_bits), case.scale, case.causal,
                                          rows=rows, rel=2.0 ** -8, sub_abs=0.0, flush=2.0 ** -126,
                                          window=case.window, block_mask=case.block_mask)
    return float((D + R + 2.0 ** -9 * np.abs(o_ref)).mean()) + 1e-6
