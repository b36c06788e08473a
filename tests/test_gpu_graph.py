"""HIP graph capture of the C-ABI calls.

The library only enqueues kernels on the caller's stream: it never allocates,
clears memory (no memset nodes) or synchronises. So every entry point can be
captured in a graph. Each replay must reproduce the eager results bit for bit
(the kernels are deterministic). The outputs are overwritten with NaN by eager
work, and the device synchronised, before every replay."""
import math

import numpy as np
import pytest
import torch

import gen
from fa_cases import say, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    import exact_attention_03_amd as fa
    dev = torch.device("cuda:0")
    B, Hq, Hkv, N, d = 1, 8, 2, 300, 128
    scale = float(np.float32(1.0 / math.sqrt(d)))
    say("graph capture: prefill/window/backward (plain, windowed)/fp8 %dx%dx%dx%dx%d, block-sparse forward and backward "
        "1x8x1x2100x128, paged decode (plain, allocation-free) and chunked prefill (plain, windowed)" % (B, Hq, Hkv, N, d))
    q = to_dev_bf16(gen.normal_bf16(181, gen.STREAM_Q, (B, Hq, N, d)))
    k = to_dev_bf16(gen.normal_bf16(181, gen.STREAM_K, (B, Hkv, N, d)))
    v = to_dev_bf16(gen.normal_bf16(181, gen.STREAM_V, (B, Hkv, N, d)))
    dout = to_dev_bf16(gen.normal_bf16(181, gen.STREAM_DO, (B, Hq, N, d)))
    o, ow, o8 = (torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    lse, lw, l8 = (torch.empty((B, Hq, N), dtype=torch.float32, device=dev) for _ in range(3))
    gq, gqw = torch.empty_like(q), torch.empty_like(q)
    gk, gv, gkw, gvw = torch.empty_like(k), torch.empty_like(v), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa.fa_backward_workspace_size(B, Hq, N), dtype=torch.uint8, device=dev)
    bwsw = torch.empty(fa.fa_backward_workspace_size(B, Hq, N), dtype=torch.uint8, device=dev)
    # block-sparse pair: 8 query heads on one K/V head, N = 2100, so the
    # dK/dV work of a key block (8 x 33 steps) is cut into runs and combined
    N2 = 2100
    q2 = to_dev_bf16(gen.normal_bf16(184, gen.STREAM_Q, (1, 8, N2, d)))
    k2 = to_dev_bf16(gen.normal_bf16(184, gen.STREAM_K, (1, 1, N2, d)))
    v2 = to_dev_bf16(gen.normal_bf16(184, gen.STREAM_V, (1, 1, N2, d)))
    do2 = to_dev_bf16(gen.normal_bf16(184, gen.STREAM_DO, (1, 8, N2, d)))
    m2 = torch.from_numpy(gen.random_block_mask(184, (1, 8, -(-N2 // 128), -(-N2 // 128)), 70)).to(dev)
    o2 = torch.empty_like(q2)
    l2 = torch.empty((1, 8, N2), dtype=torch.float32, device=dev)
    g2q, g2k, g2v = torch.empty_like(q2), torch.empty_like(k2), torch.empty_like(v2)
    sws = torch.empty(fa.fa_backward_block_sparse_workspace_size(1, 8, 1, N2, N2, d), dtype=torch.uint8, device=dev)
    assert sws.numel() > fa.fa_backward_workspace_size(1, 8, N2)  # runs and partials in use
    cq, ck, cv = (torch.empty(x.shape, dtype=torch.uint8, device=dev) for x in (q, k, v))
    sq = torch.empty((B, Hq, -(-N // 128)), device=dev)
    sk = torch.empty((B, Hkv, -(-N // 128)), device=dev)
    sv = torch.empty((B, Hkv, 1), device=dev)

    lens = [40, 2100, 700]
    sl, table, total = gen.decode_layout(182, len(lens), 1, 2100, 16, seq_lens=lens)
    max_seq_len = 2100
    qd = to_dev_bf16(gen.normal_bf16(182, gen.STREAM_Q, (len(lens), Hq, d)))
    kp = to_dev_bf16(gen.normal_bf16(182, gen.STREAM_K, (total, Hkv, 16, d)))
    vp = to_dev_bf16(gen.normal_bf16(182, gen.STREAM_V, (total, Hkv, 16, d)))
    bt, sld = torch.from_numpy(table).to(dev), torch.from_numpy(sl).to(dev)
    od, od2 = (torch.empty((len(lens), Hq, d), dtype=torch.bfloat16, device=dev) for _ in range(2))
    ld, ld2 = (torch.empty((len(lens), Hq), dtype=torch.float32, device=dev) for _ in range(2))
    dws = torch.empty(fa.fa_paged_decode_workspace_size(len(lens), Hq, d, 16, max_seq_len), dtype=torch.uint8,
                      device=dev)
    cu = torch.tensor([0, 20, 220, 320], dtype=torch.int32, device=dev)
    qp = to_dev_bf16(gen.normal_bf16(183, gen.STREAM_Q, (320, Hq, d)))
    op = torch.empty((320, Hq, d), dtype=torch.bfloat16, device=dev)
    lp = torch.empty((320, Hq), dtype=torch.float32, device=dev)
    opw = torch.empty((320, Hq, d), dtype=torch.bfloat16, device=dev)
    lpw = torch.empty((320, Hq), dtype=torch.float32, device=dev)

    def calls():
        fa.fa_forward(q, k, v, o, lse, True, scale)
        fa.fa_forward_window(q, k, v, ow, lw, True, 64, -1, scale)
        fa.fa_backward(q, k, v, o, lse, dout, gq, gk, gv, True, scale, bws)
        fa.fa_backward_window(q, k, v, ow, lw, dout, gqw, gkw, gvw, True, 64, -1, scale, bwsw)
        fa.fa_forward_block_sparse(q2, k2, v2, o2, l2, True, m2, scale)
        fa.fa_backward_block_sparse(q2, k2, v2, o2, l2, do2, g2q, g2k, g2v, True, m2, scale, sws)
        fa.fa_quantize_fp8(q, cq, sq, 128)
        fa.fa_quantize_fp8(k, ck, sk, 128)
        fa.fa_quantize_fp8(v, cv, sv, N)
        fa.fa_forward_fp8(cq, sq, ck, sk, cv, sv.reshape(B, Hkv), o8, l8, True, scale)
        fa.fa_paged_decode(qd, kp, vp, bt, sld, od, ld, max_seq_len, scale, dws)
        fa.fa_paged_decode_noalloc(qd, kp, vp, bt, sld, od2, ld2, max_seq_len, scale)
        fa.fa_paged_prefill(qp, kp, vp, bt, sld, cu, op, lp, 200, True, scale)
        fa.fa_paged_prefill_window(qp, kp, vp, bt, sld, cu, opw, lpw, 200, True, 300, -1, scale)

    outs = [o, lse, ow, lw, gq, gk, gv, gqw, gkw, gvw, o2, l2, g2q, g2k, g2v, cq, ck, cv, sq, sk, sv, o8, l8, od, ld,
            od2, ld2, op, lp, opw, lpw]
    calls()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()

    for rep in range(3):
        for x in outs:  # eager work between replays
            if x.dtype == torch.uint8:
                x.fill_(0x7F)
            else:
                x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (x, r) in enumerate(zip(outs, ref)):
            same = torch.equal(x.view(torch.uint8), r.view(torch.uint8))
            assert same, "replay %d: output %d differs from the eager run" % (rep, i)
    say("  %d outputs bit-identical to the eager run on 3 replays" % len(outs))
