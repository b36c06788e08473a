"""The C ABI without a GPU: libfa.so loads, exports every function include/fa.h
declares, and rejects every invalid argument with its status code before any
HIP call (so these run on a machine with no GPU)."""
import ctypes
import os
import re

import pytest

import exact_attention_03_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: validation fails before any launch


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    names = declared_functions()
    assert names == ["fa_backward", "fa_backward_block_sparse", "fa_backward_block_sparse_workspace_size",
                     "fa_backward_window", "fa_backward_workspace_size",
                     "fa_forward",
                     "fa_forward_block_sparse",
                     "fa_forward_fp8", "fa_forward_window", "fa_paged_decode", "fa_paged_decode_noalloc",
                     "fa_paged_decode_workspace_size",
                     "fa_paged_prefill", "fa_paged_prefill_window", "fa_quantize_fp8", "fa_quantize_fp8_incoherent",
                     "fa_status_string"]
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for st, name in fa.STATUS_NAMES.items():
        assert fa.fa_status_string(st)
    assert fa.fa_status_string(12345) == "unknown status"


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Nq=16, Nk=16, d=128,
             causal=1, scale=0.088, stream=None)
    a.update(kw)
    return fa.load().fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(B=-1), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2),
    (dict(Nq=-1), -2), (dict(Nk=-5), -2), (dict(Nq=1 << 30), -2),
    (dict(B=1 << 20, Hq=64, Hkv=8, Nq=1 << 20, d=128), -2),
    (dict(Hq=8, Hkv=3), -3), (dict(Hq=4, Hkv=8), -3),
    (dict(d=96), -4), (dict(d=256), -4), (dict(d=0), -4),
    (dict(scale=0.0), -7), (dict(scale=-1.0), -7), (dict(scale=float("inf")), -7), (dict(scale=float("nan")), -7),
])
def test_forward_rejects_invalid_arguments(kw, status):
    assert fwd(**kw) == status


def test_forward_empty_query_is_a_noop():
    # Nq == 0 returns FA_OK without touching the (null) buffers.
    assert fwd(q=None, o=None, lse=None, k=None, v=None, Nq=0) == 0


def test_forward_nk_zero_needs_no_kv_pointers_but_reaches_launch():
    # Valid arguments get past validation; without a GPU the enqueue fails
    # with FA_ERR_HIP rather than silently doing something else.
    st = fwd(k=None, v=None, Nk=0)
    assert st in (0, -100)


def dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, ps=16, o=FAKE, lse=FAKE, B=4, Hq=64, Hkv=8, d=128,
             num_pages=100, maxp=64, max_seq_len=1024, scale=0.088, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return fa.load().fa_paged_decode(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["ps"], a["o"], a["lse"],
                                     a["B"], a["Hq"], a["Hkv"], a["d"], a["num_pages"], a["maxp"],
                                     a["max_seq_len"], a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(bt=None), -1), (dict(sl=None), -1),
    (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=-1), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(num_pages=0), -2), (dict(maxp=0), -2),
    (dict(max_seq_len=0), -2), (dict(max_seq_len=1025, maxp=64), -2),
    (dict(Hq=64, Hkv=7), -3), (dict(d=80), -4), (dict(ps=32), -5), (dict(ps=8), -5),
    (dict(ws=None), -6), (dict(ws_bytes=100), -6), (dict(scale=0.0), -7),
])
def test_decode_rejects_invalid_arguments(kw, status):
    assert dec(**kw) == status


def test_decode_empty_batch_is_a_noop():
    assert dec(B=0, q=None, o=None, lse=None, ws=None, ws_bytes=0) == 0


def dec_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, ps=16, o=FAKE, lse=FAKE, B=4, Hq=64, Hkv=8, d=128,
             num_pages=100, maxp=64, max_seq_len=1024, scale=0.088, stream=None)
    a.update(kw)
    return fa.load().fa_paged_decode_noalloc(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["ps"], a["o"], a["lse"],
                                             a["B"], a["Hq"], a["Hkv"], a["d"], a["num_pages"], a["maxp"],
                                             a["max_seq_len"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(bt=None), -1), (dict(sl=None), -1), (dict(lse=None), -1),
    (dict(B=-1), -2), (dict(Hq=0), -2), (dict(num_pages=0), -2), (dict(max_seq_len=1025, maxp=64), -2),
    (dict(Hq=64, Hkv=7), -3), (dict(d=80), -4), (dict(ps=32), -5), (dict(scale=0.0), -7),
    # partials past the 32 MiB scratch: 128 sequences x 64 heads x 8 splits of 4096 x 129 floats
    (dict(B=128, num_pages=300000, maxp=2048, max_seq_len=32768), -6),
    (dict(B=32, Hq=64, Hkv=64, d=64, num_pages=300000, maxp=8192, max_seq_len=131072), -6),
])
def test_decode_noalloc_rejects_invalid_arguments(kw, status):
    """Every rejection happens before any HIP call, the scratch size check
    included."""
    assert dec_noalloc(**kw) == status


def test_decode_noalloc_empty_batch_is_a_noop():
    assert dec_noalloc(B=0, q=None, o=None, lse=None) == 0


def test_workspace_size():
    ws = fa.fa_paged_decode_workspace_size
    assert ws(64, 64, 128, 16, 32768) == 64 * 64 * 16 * 129 * 4   # 2048-token splits
    assert ws(1, 1, 64, 16, 1) == 1 * 1 * 1 * 65 * 4
    assert ws(1, 1, 96, 16, 100) == 0 and ws(1, 1, 128, 8, 100) == 0 and ws(1, 0, 128, 16, 10) == 0
    prev = 0
    for L in [1, 1023, 1024, 1025, 5000, 32768, 65536]:
        cur = ws(8, 16, 128, 16, L)
        assert cur >= prev
        prev = cur
    assert ws(9, 16, 128, 16, 5000) >= ws(8, 16, 128, 16, 5000)
    assert ws(8, 32, 128, 16, 5000) >= ws(8, 16, 128, 16, 5000)
    assert ws(8, 16, 128, 16, 5000) >= ws(8, 16, 64, 16, 5000)


def pre(windowed=False, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, ps=16, o=FAKE, lse=FAKE, B=4, Hq=64, Hkv=8,
             d=128, num_pages=100, maxp=64, max_q_len=512, causal=1, left=100, right=-1, scale=0.088, stream=None)
    a.update(kw)
    head = (a["q"], a["k"], a["v"], a["bt"], a["sl"], a["cu"], a["ps"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
            a["d"], a["num_pages"], a["maxp"], a["max_q_len"], a["causal"])
    if windowed:
        return fa.load().fa_paged_prefill_window(*head, a["left"], a["right"], a["scale"], a["stream"])
    return fa.load().fa_paged_prefill(*head, a["scale"], a["stream"])


@pytest.mark.parametrize("windowed", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(bt=None), -1), (dict(sl=None), -1),
    (dict(cu=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=-1), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(num_pages=0), -2), (dict(maxp=0), -2),
    (dict(max_q_len=-1), -2), (dict(max_q_len=1 << 30), -2), (dict(maxp=1 << 27), -2),
    (dict(Hq=64, Hkv=7), -3), (dict(d=80), -4), (dict(ps=32), -5),
    (dict(scale=0.0), -7), (dict(scale=float("nan")), -7),
])
def test_paged_prefill_rejects_invalid_arguments(windowed, kw, status):
    assert pre(windowed, **kw) == status


@pytest.mark.parametrize("kw", [dict(left=-2), dict(right=-2), dict(left=-5, right=-5),
                                dict(left=-2, B=0, q=None, o=None, lse=None)])
def test_paged_prefill_window_rejects_bad_bounds(kw):
    assert pre(True, **kw) == -8


@pytest.mark.parametrize("windowed", [False, True])
def test_paged_prefill_empty_is_a_noop(windowed):
    assert pre(windowed, B=0, q=None, o=None, lse=None) == 0
    assert pre(windowed, max_q_len=0, q=None, o=None, lse=None) == 0


def win(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Nq=16, Nk=16, d=128,
             causal=1, left=4, right=-1, scale=0.088, stream=None)
    a.update(kw)
    return fa.load().fa_forward_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                       a["Nq"], a["Nk"], a["d"], a["causal"], a["left"], a["right"], a["scale"],
                                       a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(B=0), -2), (dict(Hq=8, Hkv=3), -3), (dict(d=96), -4), (dict(scale=0.0), -7),
    (dict(left=-2), -8), (dict(right=-5), -8),
])
def test_forward_window_rejects_invalid_arguments(kw, status):
    assert win(**kw) == status


def test_forward_window_empty_query_is_a_noop():
    assert win(q=None, o=None, lse=None, k=None, v=None, Nq=0) == 0


def sparse(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Nq=16, Nk=16, d=128,
             causal=1, mask=FAKE, sb=0, sh=0, scale=0.088, stream=None)
    a.update(kw)
    return fa.load().fa_forward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                             a["Nq"], a["Nk"], a["d"], a["causal"], a["mask"], a["sb"], a["sh"],
                                             a["scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(mask=None), -1), (dict(B=0), -2), (dict(Hq=8, Hkv=3), -3), (dict(d=96), -4),
    (dict(scale=0.0), -7), (dict(sb=-1), -2), (dict(sh=-4), -2),
    (dict(Nk=4096 * 128 + 1), -2),
])
def test_forward_block_sparse_rejects_invalid_arguments(kw, status):
    assert sparse(**kw) == status


def test_forward_block_sparse_limits_match_the_header():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    assert re.search(r"#define FA_SPARSE_BLOCK 128\b", src)
    assert re.search(r"#define FA_SPARSE_MAX_KEY_BLOCKS 4096\b", src)
    assert re.search(r"#define FA_SPARSE_MAX_BACKWARD_STEPS 131072\b", src)
    assert fa.SPARSE_BLOCK == 128


def test_forward_block_sparse_empty_query_is_a_noop():
    assert sparse(q=None, o=None, lse=None, k=None, v=None, mask=None, Nq=0) == 0


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=8, Hkv=2,
             Nq=16, Nk=16, d=128, causal=1, scale=0.088, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return fa.load().fa_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                 a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                                 a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(do=None), -1), (dict(dq=None), -1),
    (dict(dk=None), -1), (dict(dv=None), -1), (dict(k=None), -1),
    (dict(B=0), -2), (dict(Nq=-1), -2), (dict(Hq=8, Hkv=3), -3), (dict(d=96), -4), (dict(scale=0.0), -7),
    (dict(ws=None), -6), (dict(ws_bytes=8 * 16 * 4 - 1), -6),
])
def test_backward_rejects_invalid_arguments(kw, status):
    assert bwd(**kw) == status


def test_backward_workspace_size():
    assert fa.fa_backward_workspace_size(2, 8, 100) == 2 * 8 * 100 * 8
    assert fa.fa_backward_workspace_size(1, 0, 10) == 0
    assert fa.fa_backward_workspace_size(-1, 4, 10) == 0
    # exactly the size passes the workspace check (a null q is then what is reported)
    assert bwd(ws_bytes=8 * 16 * 8, B=1, Hq=8, dq=None) == -1
    assert bwd(ws_bytes=8 * 16 * 8 - 1, B=1, Hq=8, dq=FAKE) == -6


def test_backward_empty_is_a_noop():
    assert bwd(Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
               ws=None) == 0


def bwdw(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=8, Hkv=2,
             Nq=16, Nk=16, d=128, causal=1, left=32, right=-1, scale=0.088, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return fa.load().fa_backward_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                        a["dv"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"],
                                        a["left"], a["right"], a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(do=None), -1), (dict(dk=None), -1), (dict(B=0), -2), (dict(Hq=8, Hkv=3), -3),
    (dict(d=96), -4), (dict(scale=float("inf")), -7), (dict(ws=None), -6), (dict(left=-2), -8),
    (dict(right=-5, causal=0), -8),
])
def test_backward_window_rejects_invalid_arguments(kw, status):
    assert bwdw(**kw) == status


def test_backward_window_empty_is_a_noop():
    assert bwdw(Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                ws=None) == 0


def bwds(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=8, Hkv=2,
             Nq=16, Nk=16, d=128, causal=1, mask=FAKE, sb=0, sh=0, scale=0.088, ws=FAKE, ws_bytes=1 << 20,
             stream=None)
    a.update(kw)
    return fa.load().fa_backward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                              a["dv"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                              a["causal"], a["mask"], a["sb"], a["sh"], a["scale"], a["ws"],
                                              a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(mask=None), -1), (dict(do=None), -1), (dict(dq=None), -1), (dict(dk=None), -1),
    (dict(dv=None), -1), (dict(B=0), -2), (dict(Hq=8, Hkv=3), -3), (dict(d=96), -4), (dict(scale=0.0), -7),
    (dict(sb=-1), -2), (dict(sh=-4), -2), (dict(Nk=4096 * 128 + 1), -2), (dict(ws=None), -6),
    (dict(ws_bytes=8 * 16 * 8 - 1), -6),
])
def test_backward_block_sparse_rejects_invalid_arguments(kw, status):
    assert bwds(**kw) == status


def test_backward_block_sparse_workspace_size():
    # one run per key block: exactly fa_backward's workspace
    assert fa.fa_backward_block_sparse_workspace_size(1, 8, 2, 1000, 1000, 128) == 8 * 1000 * 8
    # causal GQA 64/8 N=8192: a key block's 8 x 128 steps may be cut into two
    # runs: rows, then 8 x 64 x 2 fp32 partials of 2 x 128 x 128, a flag per
    # partial and a run count per key block
    slots = 8 * 64 * 2
    assert fa.fa_backward_block_sparse_workspace_size(1, 64, 8, 8192, 8192, 128) == \
        64 * 8192 * 8 + slots * 2 * 128 * 128 * 4 + slots * 4 + 8 * 64 * 4
    # at most FA_SPARSE_MAX_BACKWARD_STEPS steps per key block
    assert fa.fa_backward_block_sparse_workspace_size(1, 8, 1, 64 * 16384, 128, 64) > 0
    assert fa.fa_backward_block_sparse_workspace_size(1, 8, 1, 64 * 16384 + 1, 128, 64) == 0
    assert bwds(Hq=8, Hkv=1, Nq=64 * 16384 + 1, Nk=128) == -2
    # B * Hkv >= 16: never cut
    assert fa.fa_backward_block_sparse_workspace_size(2, 64, 8, 8192, 8192, 128) == 2 * 64 * 8192 * 8
    for bad in [(1, 8, 3, 100, 100, 128), (1, 0, 1, 10, 10, 128), (1, 8, 2, -1, 10, 128), (1, 8, 2, 10, 10, 96),
                (0, 8, 2, 10, 10, 128)]:
        assert fa.fa_backward_block_sparse_workspace_size(*bad) == 0, bad
    need = fa.fa_backward_block_sparse_workspace_size(1, 64, 8, 8192, 8192, 128)
    assert bwds(Hq=64, Hkv=8, Nq=8192, Nk=8192, ws_bytes=need - 1) == -6
    assert bwds(Hq=64, Hkv=8, Nq=8192, Nk=8192, ws_bytes=need, dq=None) == -1


def test_backward_block_sparse_empty_is_a_noop():
    assert bwds(Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                mask=None, ws=None) == 0


def fp8(**kw):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, v=FAKE, vs=FAKE, o=FAKE, lse=FAKE, B=1, Hq=8, Hkv=2, Nq=16, Nk=16,
             d=128, causal=1, scale=0.088, stream=None)
    a.update(kw)
    return fa.load().fa_forward_fp8(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["o"], a["lse"], a["B"],
                                    a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(qs=None), -1), (dict(ks=None), -1), (dict(vs=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(Hq=8, Hkv=3), -3), (dict(d=96), -4), (dict(scale=0.0), -7),
])
def test_forward_fp8_rejects_invalid_arguments(kw, status):
    assert fp8(**kw) == status


def test_quantize_fp8_rejects_invalid_arguments():
    lib = fa.load()
    assert lib.fa_quantize_fp8(FAKE, FAKE, FAKE, 0, 1, 8, 128, 128, None) == -2
    assert lib.fa_quantize_fp8(FAKE, FAKE, FAKE, 1, 1, 8, 128, 0, None) == -2
    assert lib.fa_quantize_fp8(FAKE, FAKE, FAKE, 1, 1, 8, 96, 128, None) == -4
    assert lib.fa_quantize_fp8(None, FAKE, FAKE, 1, 1, 8, 128, 128, None) == -1
    assert lib.fa_quantize_fp8(None, None, None, 1, 1, 0, 128, 128, None) == 0
    assert fa.FP8_SCALE_ROWS == 128
    q = lib.fa_quantize_fp8_incoherent
    assert q(FAKE, FAKE, FAKE, FAKE, 0, 1, 8, 128, 128, None) == -2
    assert q(FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 128, 0, None) == -2
    assert q(FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 96, 128, None) == -4
    assert q(FAKE, None, FAKE, FAKE, 1, 1, 8, 128, 128, None) == -1
    assert q(None, FAKE, FAKE, FAKE, 1, 1, 8, 64, 128, None) == -1
    assert q(None, None, None, None, 1, 1, 0, 128, 128, None) == 0
    assert re.search(r"#define FA_FP8_SCALE_ROWS 128\b", open(os.path.join(ROOT, "include", "fa.h")).read())


def test_library_is_built_from_the_current_sources():
    """The in-tree libfa.so carries the hash of the sources it was built from;
    load() refuses a library whose sources changed since."""
    assert not fa.is_stale()
