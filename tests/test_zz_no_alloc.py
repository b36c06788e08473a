"""fa_paged_decode_noalloc (the decode with the library's own per-device
scratch, for callers that cannot allocate) against fa_paged_decode with a
caller workspace: two calls in a row through the C ABI, the second with a
smaller input and another split layout, each bit-identical to the workspace
entry point (same kernels) and within the acceptance bar of the oracle."""
import numpy as np
import pytest
import torch

import exact_attention_03_amd as fa
from fa_cases import DecodeCase, bf16_dev_to_f64, compare, say, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run_noalloc(case):
    q = to_dev_bf16(case.q_bits)
    kp, vp = to_dev_bf16(case.k_bits), to_dev_bf16(case.v_bits)
    bt = torch.from_numpy(case.table).cuda()
    sl = torch.from_numpy(case.seq_lens).cuda()
    o = torch.full((case.B, case.Hq, case.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.B, case.Hq), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_paged_decode_noalloc(q, kp, vp, bt, sl, o, lse, case.max_seq_len, case.scale, page_size=case.ps)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_decode_matches_workspace_decode(order, gpu_lib):
    # 1) the 64-sequence decode workload (4096-token splits, 16.9 MB of partials)
    big = DecodeCase(64, 64, 8, 128, seed=1005, len_lo=512, len_hi=32768, max_pages_per_seq=2048,
                     max_seq_len=32768)
    # 2) a smaller call with d = 64 (2048-token splits, another layout of the scratch)
    small = DecodeCase(5, 16, 4, 64, seed=301, seq_lens=[1, 17, 2048, 2049, 5000])
    for what, case in (("large", big), ("small", small)):
        say("noalloc decode %s: B=%d Hq=%d Hkv=%d d=%d max_seq_len=%d" % (what, case.B, case.Hq, case.Hkv, case.d,
                                                                          case.max_seq_len))
        o1, l1 = _run_noalloc(case)
        o2, l2 = case.run_gpu()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), what
        assert torch.equal(l1, l2), what
        if what == "small":
            o_ref, l_ref = case.oracle()
            compare(bf16_dev_to_f64(o1), l1.cpu().numpy().astype(np.float64), o_ref, l_ref, "noalloc " + what)


def test_noalloc_decode_rejects_sizes_past_its_scratch(gpu_lib):
    case = DecodeCase(2, 64, 8, 128, seed=302, seq_lens=[10, 20])
    q = to_dev_bf16(np.zeros((128, 64, 128), dtype=np.uint16))
    kp, vp = to_dev_bf16(case.k_bits), to_dev_bf16(case.v_bits)
    bt = torch.zeros((128, 2048), dtype=torch.int32, device="cuda")
    sl = torch.ones((128,), dtype=torch.int32, device="cuda")
    o = torch.empty((128, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((128, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_paged_decode_noalloc(q, kp, vp, bt, sl, o, lse, 32768, case.scale)
    assert e.value.status == -6
