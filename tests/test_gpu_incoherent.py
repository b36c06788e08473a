"""GPU parity of fa_quantize_fp8_incoherent (incoherent processing fused
with the FP8 block quantization) through the C ABI, against the oracle.

Page: "FlashAttention" glossary (polydesk.ai), section "FlashAttention-3":
FP8 with block quantization and incoherent processing.

The kernel transforms each row in float32 (a fast Walsh-Hadamard transform
of log2(d) butterfly stages, then 1 / sqrt(d)); the oracle computes the
transform exactly (float64). So the comparison allows what float32 can
change, and no more:
  * |y_kernel - y| <= eps = 2 ((log2(d) + 1) u sum|x| / sqrt(d) + 3 u |y|),
    u = 2^-24 (each stage adds or subtracts two rounded values whose
    magnitudes are bounded by the partial sums of |x|; then one product with
    the rounded constant);
  * the block scale: |448 scale - amax(|y|)| <= max eps + 4 u amax;
  * each code: with t = y / scale (the kernel's scale) and delta = eps / scale
    + 2 u |t|, the code's value lies between E4M3(t - delta) and
    E4M3(t + delta). Where those two agree the code is unique and must be
    that one; the elements where they differ (t within delta of a rounding
    midpoint; mostly small values, since eps follows the row's sum of |x|)
    are counted and must stay below 1%, so the check binds;
  * the codes may differ from the oracle's own float32 decision (quantize_fp8
    of y rounded once to float32) at no more than 0.1% of the elements.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from fa_cases import bf16_dev_to_f64, say, to_dev_bf16

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def gpu_quantize_incoherent(bits, signs, block):
    import exact_attention_03_amd as fa
    B, H, N, d = bits.shape
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, -(-N // block)), dtype=torch.float32, device="cuda")
    fa.fa_quantize_fp8_incoherent(to_dev_bf16(bits), torch.from_numpy(signs).cuda(), codes, scales, block)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def check_codes(x, signs, block, codes, scales, what=""):
    """x: float64 [B, H, N, d] (bf16 values); codes, scales: the kernel's.
    Returns the number of elements whose code is not unique."""
    B, H, N, d = x.shape
    L = int(np.log2(d))
    y = oracle.incoherent_transform(x, signs)
    eps = 2.0 * ((L + 1) * U * np.abs(x).sum(-1, keepdims=True) / np.sqrt(d) + 3 * U * np.abs(y))
    nb = -(-N // block)
    assert scales.shape == (B, H, nb)
    for i in range(nb):
        sl = slice(i * block, (i + 1) * block)
        amax = np.abs(y[:, :, sl]).max(axis=(2, 3))
        e = eps[:, :, sl].max(axis=(2, 3))
        s = scales[:, :, i].astype(np.float64)
        zero = amax == 0
        assert np.all(s[zero] == 1.0), what
        assert np.all(np.abs(448.0 * s[~zero] - amax[~zero]) <= e[~zero] + 4 * U * amax[~zero]), \
            "%s: block %d scale off" % (what, i)
    sc = scales.astype(np.float64)[:, :, np.arange(N) // block][..., None]
    t = y / sc
    delta = eps / sc + 2 * U * np.abs(t)
    lo = oracle.e4m3_decode(oracle.e4m3_encode(t - delta))
    hi = oracle.e4m3_decode(oracle.e4m3_encode(t + delta))
    got = oracle.e4m3_decode(codes)
    assert not np.isnan(got).any(), what
    bad = ~((got >= lo) & (got <= hi))
    assert not bad.any(), "%s: %d codes outside their float32 range, first at %s" % (
        what, int(bad.sum()), np.argwhere(bad)[0])
    amb = int((lo != hi).sum())
    ref_codes, _ = oracle.quantize_fp8_incoherent(x, signs, block)
    diff = int((oracle.e4m3_decode(ref_codes) != got).sum())
    say("  %s: %d elements, %d with two admissible codes, %d differ from the oracle's float32 decision" % (
        what, got.size, amb, diff))
    assert amb <= 1e-2 * got.size
    assert diff <= 1e-3 * got.size
    return amb


@pytest.mark.parametrize("shape", [(1, 2, 300, 128, 128), (2, 3, 129, 64, 128), (1, 1, 1000, 128, 1000),
                                   (1, 2, 64, 128, 7), (1, 3, 257, 64, 64)], ids=str)
def test_quantize_incoherent_matches_oracle(shape, gpu_lib):
    B, H, N, d, block = shape
    say("incoherent quantizer B=%d H=%d N=%d d=%d block=%d" % shape)
    bits = gen.normal_bf16(171 + N, gen.STREAM_Q, (B, H, N, d), 2.0)
    bits[0, 0, :min(N, block)] = 0                      # an all-zero block
    signs = gen.random_signs(172 + N, d)
    codes, scales = gpu_quantize_incoherent(bits, signs, block)
    check_codes(oracle.bf16_bits_to_f64(bits), signs, block, codes, scales, "normal %s" % (shape,))


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_incoherent_outlier_inputs(d, gpu_lib):
    say("incoherent quantizer, outlier inputs, d=%d" % d)
    bits = gen.outlier_bf16(181, gen.STREAM_K, (1, 4, 1000, d))
    signs = gen.random_signs(182, d)
    codes, scales = gpu_quantize_incoherent(bits, signs, 128)
    check_codes(oracle.bf16_bits_to_f64(bits), signs, 128, codes, scales, "outliers d=%d" % d)


def test_quantize_incoherent_one_hot_rows_are_exact(gpu_lib):
    # a row with one nonzero entry becomes +-v / sqrt(d) everywhere: every
    # code is +-448 and the sign pattern is s_i H[i][j]
    d, N = 128, 256
    say("incoherent quantizer, one-hot rows")
    ch = gen.uniform_int(183, gen.STREAM_PERM, N, 0, d - 1)
    x = np.zeros((1, 1, N, d))
    x[0, 0, np.arange(N), ch] = 2.0
    signs = gen.random_signs(184, d)
    from fa_cases import f64_to_bf16_bits
    codes, scales = gpu_quantize_incoherent(f64_to_bf16_bits(x), signs, 128)
    ref_codes, ref_scales = oracle.quantize_fp8_incoherent(x, signs, 128)
    np.testing.assert_array_equal(codes, ref_codes)
    np.testing.assert_array_equal(scales, ref_scales)
    h = oracle.hadamard(d)
    np.testing.assert_array_equal(np.sign(oracle.e4m3_decode(codes[0, 0])), signs[ch][:, None] * h[ch])


def test_quantize_incoherent_timed_workload_sizes(gpu_lib):
    # The FP8 workload's Q [1, 64, 8192, 128] and K [1, 8, 8192, 128] in the
    # launch the library makes for them; K checked in full, Q on three heads.
    from fa_cases import PrefillCase
    case = PrefillCase(1, 64, 8, 8192, 8192, 128, True, seed=1003)
    signs = gen.random_signs(1004, 128)
    say("incoherent quantizer, 8K workload K")
    ck, sk = gpu_quantize_incoherent(case.k_bits, signs, 128)
    check_codes(oracle.bf16_bits_to_f64(case.k_bits), signs, 128, ck, sk, "8K K")
    say("incoherent quantizer, 8K workload Q")
    cq, sq = gpu_quantize_incoherent(case.q_bits, signs, 128)
    for h in (0, 37, 63):
        check_codes(oracle.bf16_bits_to_f64(case.q_bits[:, h:h + 1]), signs, 128, cq[:, h:h + 1], sq[:, h:h + 1],
                    "8K Q head %d" % h)


def test_forward_fp8_on_incoherent_codes(gpu_lib):
    # The FP8 forward on Q and K quantized by the oracle after the transform
    # (outlier inputs, GQA, ragged, causal), under the FP8 forward's own bar.
    from test_gpu_parity import check_fp8
    B, Hq, Hkv, N, d = 1, 8, 2, 1000, 128
    f = oracle.bf16_bits_to_f64
    q = f(gen.outlier_bf16(191, gen.STREAM_Q, (B, Hq, N, d)))
    k = f(gen.outlier_bf16(191, gen.STREAM_K, (B, Hkv, N, d)))
    v = f(gen.outlier_bf16(191, gen.STREAM_V, (B, Hkv, N, d)))
    signs = gen.random_signs(192, d)
    check_fp8(B, Hq, Hkv, N, N, d, True, seed=191,
              inputs=(oracle.incoherent_transform(q, signs), oracle.incoherent_transform(k, signs), v))


def test_incoherent_path_lowers_fp8_error_on_outliers(gpu_lib):
    # The library end to end (quantizers + FP8 forward) against exact
    # attention of the bf16 inputs: block scales with incoherent processing
    # against one scale per head and tensor without it, the comparison the
    # page makes. The oracle's pin of the same recipe gives 1.45-1.62x.
    import exact_attention_03_amd as fa
    B, H, N, d = 1, 2, 512, 128
    bits = [gen.outlier_bf16(203, st, (B, H, N, d)) for st in (gen.STREAM_Q, gen.STREAM_K, gen.STREAM_V)]
    q, k, v = (oracle.bf16_bits_to_f64(b) for b in bits)
    scale = float(np.float32(1 / np.sqrt(d)))
    ref, _ = oracle.attention_naive(q, k, v, scale, False)
    signs = gen.random_signs(204, d)
    dq, dk, dv = (to_dev_bf16(b) for b in bits)
    nb = N // 128
    cv = torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda")
    sv = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
    fa.fa_quantize_fp8(dv, cv, sv, N)

    def run(incoherent):
        cq = torch.empty((B, H, N, d), dtype=torch.uint8, device="cuda")
        ck = torch.empty_like(cq)
        if incoherent:
            sq = torch.empty((B, H, nb), dtype=torch.float32, device="cuda")
            sk = torch.empty_like(sq)
            sg = torch.from_numpy(signs).cuda()
            fa.fa_quantize_fp8_incoherent(dq, sg, cq, sq, 128)
            fa.fa_quantize_fp8_incoherent(dk, sg, ck, sk, 128)
        else:  # one scale per (batch, head), repeated over the forward's 128-row blocks
            sq1 = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
            sk1 = torch.empty_like(sq1)
            fa.fa_quantize_fp8(dq, cq, sq1, N)
            fa.fa_quantize_fp8(dk, ck, sk1, N)
            sq, sk = sq1.expand(B, H, nb).contiguous(), sk1.expand(B, H, nb).contiguous()
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        fa.fa_forward_fp8(cq, sq, ck, sk, cv, sv.reshape(B, H), o, lse, False, scale)
        torch.cuda.synchronize()
        return float(np.sqrt(np.mean((bf16_dev_to_f64(o) - ref) ** 2)))

    say("incoherent vs per-tensor FP8 on outlier inputs")
    base, inc = run(False), run(True)
    say("  O rmse against exact attention: per-tensor %.4e, block + incoherent %.4e, ratio %.2f" % (
        base, inc, base / inc))
    assert base / inc > 1.3
