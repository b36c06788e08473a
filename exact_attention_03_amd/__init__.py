"""Python binding of libfa (exact attention forward for MI355X / gfx950).

Argument marshalling only: every function below checks that torch tensors
have the dtype, device, contiguity and shapes the C ABI (include/fa.h)
expects, passes their device pointers and the caller's HIP stream to the
library, and raises FAError on a non-zero status. All arithmetic runs in the
library's HIP kernels; there is no other implementation to fall back to, and
a missing library raises instead of computing anything.

Functions (same names as the C ABI):
  fa_forward(q, k, v, o, lse, causal, scale, stream=None)
  fa_forward_window(q, k, v, o, lse, causal, window_left, window_right, scale, stream=None)
  fa_forward_block_sparse(q, k, v, o, lse, causal, block_mask, scale, stream=None)
  fa_quantize_fp8(x, codes, scales, block_rows, stream=None)
  fa_quantize_fp8_incoherent(x, signs, codes, scales, block_rows, stream=None)
  fa_forward_fp8(q, q_scales, k, k_scales, v, v_scales, o, lse, causal, scale, stream=None)
  fa_backward_workspace_size(B, Hq, Nq)
  fa_backward(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace, stream=None)
  fa_backward_window(q, k, v, o, lse, dout, dq, dk, dv, causal, window_left, window_right, scale, workspace,
                     stream=None)
  fa_backward_block_sparse_workspace_size(B, Hq, Hkv, Nq, Nk, d)
  fa_backward_block_sparse(q, k, v, o, lse, dout, dq, dk, dv, causal, block_mask, scale, workspace, stream=None)
  fa_paged_decode_workspace_size(B, Hq, d, page_size, max_seq_len)
  fa_paged_decode(q, k_pool, v_pool, block_table, seq_lens, o, lse,
                  max_seq_len, scale, workspace, page_size=16, stream=None)
  fa_paged_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, o, lse,
                          max_seq_len, scale, page_size=16, stream=None)
  fa_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse,
                   max_q_len, causal, scale, page_size=16, stream=None)
  fa_paged_prefill_window(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse,
                          max_q_len, causal, window_left, window_right, scale, page_size=16, stream=None)
  fa_status_string(status)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
_DEFAULT_LIB = LIB_PATH

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_GQA",
                -4: "FA_ERR_HEADDIM", -5: "FA_ERR_PAGESIZE", -6: "FA_ERR_WORKSPACE",
                -7: "FA_ERR_SCALE", -8: "FA_ERR_WINDOW", -100: "FA_ERR_HIP"}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (what, STATUS_NAMES.get(status, status),
                                                 fa_status_string(status)))


def is_stale() -> bool:
    """True when the in-tree libfa.so was not built from the sources as they
    are now (its stamp, written by the build, holds their hash)."""
    from . import _build
    try:
        with open(_build.STAMP) as fh:
            return fh.read().strip() != _build.source_digest()
    except OSError:
        return True


def load() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_attention_03_amd._build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfa.so is not built (%s); run `python -m exact_attention_03_amd._build`"
                          % LIB_PATH)
    if LIB_PATH == _DEFAULT_LIB and is_stale():
        raise ImportError("libfa.so is older than its sources (%s); rebuild with "
                          "`python -m exact_attention_03_amd._build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.fa_forward.restype = i32
    lib.fa_forward_window.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.fa_forward_window.restype = i32
    i64 = ctypes.c_longlong
    lib.fa_forward_block_sparse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, i64, i64,
                                            f32, vp]
    lib.fa_forward_block_sparse.restype = i32
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.fa_quantize_fp8.restype = i32
    lib.fa_quantize_fp8_incoherent.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.fa_quantize_fp8_incoherent.restype = i32
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.fa_forward_fp8.restype = i32
    lib.fa_backward_workspace_size.argtypes = [i32, i32, i32]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.fa_backward.restype = i32
    lib.fa_backward_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                       f32, vp, sz, vp]
    lib.fa_backward_window.restype = i32
    lib.fa_backward_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             vp, i64, i64, f32, vp, sz, vp]
    lib.fa_backward_block_sparse.restype = i32
    lib.fa_backward_block_sparse_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_backward_block_sparse_workspace_size.restype = sz
    lib.fa_paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_paged_decode_workspace_size.restype = sz
    lib.fa_paged_decode.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                    i32, f32, vp, sz, vp]
    lib.fa_paged_decode.restype = i32
    lib.fa_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                            i32, f32, vp]
    lib.fa_paged_decode_noalloc.restype = i32
    lib.fa_paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i32, f32, vp]
    lib.fa_paged_prefill.restype = i32
    lib.fa_paged_prefill_window.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                            i32, i32, i32, i32, f32, vp]
    lib.fa_paged_prefill_window.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _stream_ptr(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def fa_forward(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], o [B,Hq,Nq,d] (bf16), lse [B,Hq,Nq] (fp32)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(q, "q", torch.bfloat16)
    _check(k, "k", torch.bfloat16, (B, Hkv, Nk, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, Nk, d))
    _check(o, "o", torch.bfloat16, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    st = load().fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, Hq, Hkv, Nq, Nk, d, 1 if causal else 0, float(scale), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_forward")


def fa_forward_window(q, k, v, o, lse, causal: bool, window_left: int, window_right: int, scale: float,
                      stream=None) -> None:
    """As fa_forward, with a sliding window: query i (at key position
    i + Nk - Nq) sees keys in [p - window_left, p + window_right]; -1 is
    unbounded and causal forces the right bound to 0."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(q, "q", torch.bfloat16)
    _check(k, "k", torch.bfloat16, (B, Hkv, Nk, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, Nk, d))
    _check(o, "o", torch.bfloat16, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    st = load().fa_forward_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, Hq, Hkv, Nq, Nk, d, 1 if causal else 0, int(window_left),
                                  int(window_right), float(scale), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_forward_window")


SPARSE_BLOCK = 128  # queries and keys per block of a block-sparse mask


def _mask_strides(block_mask, B, Hq, Nq, Nk):
    """Batch and head strides (bytes; 0 broadcasts) of a block mask of shape
    [B or 1, Hq or 1, ceil(Nq/128), ceil(Nk/128)] whose last two dimensions
    are contiguous."""
    import torch
    if not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8:
        raise TypeError("block_mask must be a torch.uint8 tensor")
    if block_mask.device.type != "cuda":
        raise ValueError("block_mask must be on a GPU device")
    nqb, nkb = -(-Nq // SPARSE_BLOCK), -(-Nk // SPARSE_BLOCK)
    if block_mask.dim() != 4 or block_mask.shape[0] not in (1, B) or block_mask.shape[1] not in (1, Hq) or \
            tuple(block_mask.shape[2:]) != (nqb, nkb):
        raise ValueError("block_mask must have shape [%d or 1, %d or 1, %d, %d], got %s"
                         % (B, Hq, nqb, nkb, tuple(block_mask.shape)))
    if block_mask.stride(3) != 1 or block_mask.stride(2) != nkb:
        raise ValueError("block_mask's last two dimensions must be contiguous")
    sb = 0 if block_mask.shape[0] == 1 else block_mask.stride(0)
    sh = 0 if block_mask.shape[1] == 1 else block_mask.stride(1)
    return sb, sh


def fa_forward_block_sparse(q, k, v, o, lse, causal: bool, block_mask, scale: float, stream=None) -> None:
    """As fa_forward, with a block mask: block_mask is a uint8 GPU tensor of
    shape [B or 1, Hq or 1, ceil(Nq/128), ceil(Nk/128)] (a size-1 batch or
    head dimension is broadcast) whose last two dimensions are contiguous;
    nonzero entries mark the (query block, key block) pairs that attend."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(q, "q", torch.bfloat16)
    _check(k, "k", torch.bfloat16, (B, Hkv, Nk, d))
    _check(v, "v", torch.bfloat16, (B, Hkv, Nk, d))
    _check(o, "o", torch.bfloat16, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    sb, sh = _mask_strides(block_mask, B, Hq, Nq, Nk)
    st = load().fa_forward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        B, Hq, Hkv, Nq, Nk, d, 1 if causal else 0, block_mask.data_ptr(),
                                        int(sb), int(sh), float(scale), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_forward_block_sparse")


FP8_SCALE_ROWS = 128  # rows per Q / K scale block of fa_forward_fp8


def fa_quantize_fp8(x, codes, scales, block_rows: int, stream=None) -> None:
    """x [B,H,N,d] bf16 -> codes [B,H,N,d] uint8 (E4M3), scales
    [B,H,ceil(N/block_rows)] float32 (one per block of rows)."""
    import torch
    if x.dim() != 4:
        raise ValueError("x must be 4-D [batch, heads, seq, head_dim]")
    B, H, N, d = x.shape
    _check(x, "x", torch.bfloat16)
    _check(codes, "codes", torch.uint8, (B, H, N, d))
    _check(scales, "scales", torch.float32, (B, H, -(-N // max(1, block_rows))))
    st = load().fa_quantize_fp8(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H, N, d, int(block_rows),
                                _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_quantize_fp8")


def fa_quantize_fp8_incoherent(x, signs, codes, scales, block_rows: int, stream=None) -> None:
    """x [B,H,N,d] bf16, signs [d] int8 (negative: negate the channel) ->
    codes [B,H,N,d] uint8 (E4M3 of the rows times diag(signs) H_d / sqrt(d)),
    scales [B,H,ceil(N/block_rows)] float32."""
    import torch
    if x.dim() != 4:
        raise ValueError("x must be 4-D [batch, heads, seq, head_dim]")
    B, H, N, d = x.shape
    _check(x, "x", torch.bfloat16)
    _check(signs, "signs", torch.int8, (d,))
    _check(codes, "codes", torch.uint8, (B, H, N, d))
    _check(scales, "scales", torch.float32, (B, H, -(-N // max(1, block_rows))))
    st = load().fa_quantize_fp8_incoherent(x.data_ptr(), signs.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H,
                                           N, d, int(block_rows), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_quantize_fp8_incoherent")


def fa_forward_fp8(q, q_scales, k, k_scales, v, v_scales, o, lse, causal: bool, scale: float, stream=None) -> None:
    """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] uint8 E4M3 codes; q_scales
    [B,Hq,ceil(Nq/128)], k_scales [B,Hkv,ceil(Nk/128)], v_scales [B,Hkv]
    float32; o [B,Hq,Nq,d] bf16, lse [B,Hq,Nq] float32."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(q, "q", torch.uint8)
    _check(k, "k", torch.uint8, (B, Hkv, Nk, d))
    _check(v, "v", torch.uint8, (B, Hkv, Nk, d))
    _check(q_scales, "q_scales", torch.float32, (B, Hq, -(-Nq // FP8_SCALE_ROWS)))
    _check(k_scales, "k_scales", torch.float32, (B, Hkv, -(-Nk // FP8_SCALE_ROWS)))
    _check(v_scales, "v_scales", torch.float32, (B, Hkv))
    _check(o, "o", torch.bfloat16, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    st = load().fa_forward_fp8(q.data_ptr(), q_scales.data_ptr(), k.data_ptr(), k_scales.data_ptr(), v.data_ptr(),
                               v_scales.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                               1 if causal else 0, float(scale), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_forward_fp8")


def fa_backward_workspace_size(B: int, Hq: int, Nq: int) -> int:
    return int(load().fa_backward_workspace_size(B, Hq, Nq))


def _backward_shapes(q, k, v, o, lse, dout, dq, dk, dv, workspace):
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, seq, head_dim]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(q, "q", torch.bfloat16)
    for t, name in ((k, "k"), (v, "v"), (dk, "dk"), (dv, "dv")):
        _check(t, name, torch.bfloat16, (B, Hkv, Nk, d))
    for t, name in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _check(t, name, torch.bfloat16, (B, Hq, Nq, d))
    _check(lse, "lse", torch.float32, (B, Hq, Nq))
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return B, Hq, Hkv, Nq, Nk, d, workspace.numel() * workspace.element_size()


def fa_backward(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, scale: float, workspace, stream=None) -> None:
    """Gradients of fa_forward: q, o, dout, dq [B,Hq,Nq,d] bf16; k, v, dk, dv
    [B,Hkv,Nk,d] bf16; lse [B,Hq,Nq] fp32 (the forward's); workspace: a GPU
    tensor of at least fa_backward_workspace_size(B, Hq, Nq) bytes."""
    B, Hq, Hkv, Nq, Nk, d, nbytes = _backward_shapes(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    st = load().fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk, d, 1 if causal else 0,
                            float(scale), workspace.data_ptr(), nbytes, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_backward")


def fa_backward_window(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, window_left: int, window_right: int,
                       scale: float, workspace, stream=None) -> None:
    """Gradients of fa_forward_window (same window arguments); tensors as for
    fa_backward."""
    B, Hq, Hkv, Nq, Nk, d, nbytes = _backward_shapes(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    st = load().fa_backward_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nk,
                                   d, 1 if causal else 0, int(window_left), int(window_right), float(scale),
                                   workspace.data_ptr(), nbytes, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_backward_window")


def fa_backward_block_sparse_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_backward_block_sparse_workspace_size(B, Hq, Hkv, Nq, Nk, d))


def fa_backward_block_sparse(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, block_mask, scale: float, workspace,
                             stream=None) -> None:
    """Gradients of fa_forward_block_sparse (same block_mask); tensors as for
    fa_backward, workspace of fa_backward_block_sparse_workspace_size bytes."""
    B, Hq, Hkv, Nq, Nk, d, nbytes = _backward_shapes(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    sb, sh = _mask_strides(block_mask, B, Hq, Nq, Nk)
    st = load().fa_backward_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv,
                                         Nq, Nk, d, 1 if causal else 0, block_mask.data_ptr(), int(sb), int(sh),
                                         float(scale), workspace.data_ptr(), nbytes, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_backward_block_sparse")


def fa_paged_decode_workspace_size(B: int, Hq: int, d: int, page_size: int, max_seq_len: int) -> int:
    return int(load().fa_paged_decode_workspace_size(B, Hq, d, page_size, max_seq_len))


def fa_paged_decode(q, k_pool, v_pool, block_table, seq_lens, o, lse, max_seq_len: int,
                    scale: float, workspace, page_size: int = 16, stream=None) -> None:
    """q [B,Hq,d] bf16; pools [num_pages,Hkv,page_size,d] bf16; block_table
    [B,max_pages] int32; seq_lens [B] int32; o [B,Hq,d] bf16; lse [B,Hq] fp32;
    workspace: a uint8 tensor of at least fa_paged_decode_workspace_size bytes."""
    import torch
    B, Hq, d = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    _check(q, "q", torch.bfloat16)
    _check(k_pool, "k_pool", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _check(v_pool, "v_pool", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _check(block_table, "block_table", torch.int32)
    _check(seq_lens, "seq_lens", torch.int32, (B,))
    _check(o, "o", torch.bfloat16, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages_per_seq]")
    _check(workspace, "workspace", workspace.dtype)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().fa_paged_decode(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                block_table.data_ptr(), seq_lens.data_ptr(), page_size,
                                o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, num_pages,
                                block_table.shape[1], int(max_seq_len), float(scale),
                                workspace.data_ptr(), ws_bytes, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_paged_decode")


# The allocation-free decode's scratch per device (FA_PAGED_DECODE_NOALLOC_MAX_BYTES in fa.h).
PAGED_DECODE_NOALLOC_MAX_BYTES = 32 << 20


def fa_paged_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, o, lse, max_seq_len: int,
                            scale: float, page_size: int = 16, stream=None) -> None:
    """fa_paged_decode with the library's own per-device scratch instead of a
    workspace (for callers that cannot allocate); same tensors otherwise.
    Calls that overlap on one device race on that scratch."""
    import torch
    B, Hq, d = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    _check(q, "q", torch.bfloat16)
    _check(k_pool, "k_pool", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _check(v_pool, "v_pool", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _check(block_table, "block_table", torch.int32)
    _check(seq_lens, "seq_lens", torch.int32, (B,))
    _check(o, "o", torch.bfloat16, (B, Hq, d))
    _check(lse, "lse", torch.float32, (B, Hq))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages_per_seq]")
    st = load().fa_paged_decode_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                        block_table.data_ptr(), seq_lens.data_ptr(), page_size,
                                        o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, num_pages,
                                        block_table.shape[1], int(max_seq_len), float(scale), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_paged_decode_noalloc")



def _paged_prefill_shapes(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse, page_size):
    """Checks the paged prefill tensors; returns (B, Hq, Hkv, d, num_pages)."""
    import torch
    total_q, Hq, d = q.shape
    num_pages, Hkv = k_pool.shape[0], k_pool.shape[1]
    _check(q, "q", torch.bfloat16)
    _check(k_pool, "k_pool", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _check(v_pool, "v_pool", torch.bfloat16, (num_pages, Hkv, page_size, d))
    _check(block_table, "block_table", torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_pages_per_seq]")
    B = block_table.shape[0]
    _check(seq_lens, "seq_lens", torch.int32, (B,))
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, (B + 1,))
    _check(o, "o", torch.bfloat16, (total_q, Hq, d))
    _check(lse, "lse", torch.float32, (total_q, Hq))
    return B, Hq, Hkv, d, num_pages


def fa_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse, max_q_len: int,
                     causal: bool, scale: float, page_size: int = 16, stream=None) -> None:
    """q [total_q,Hq,d] bf16 (packed rows); pools [num_pages,Hkv,page_size,d]
    bf16; block_table [B,max_pages] int32; seq_lens [B] int32;
    cu_seqlens_q [B+1] int32; o [total_q,Hq,d] bf16; lse [total_q,Hq] fp32."""
    B, Hq, Hkv, d, num_pages = _paged_prefill_shapes(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o,
                                                     lse, page_size)
    st = load().fa_paged_prefill(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                 block_table.data_ptr(), seq_lens.data_ptr(), cu_seqlens_q.data_ptr(),
                                 page_size, o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, num_pages,
                                 block_table.shape[1], int(max_q_len), 1 if causal else 0, float(scale),
                                 _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_paged_prefill")


def fa_paged_prefill_window(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse, max_q_len: int,
                            causal: bool, window_left: int, window_right: int, scale: float, page_size: int = 16,
                            stream=None) -> None:
    """fa_paged_prefill with a sliding window; -1 leaves a bound open."""
    B, Hq, Hkv, d, num_pages = _paged_prefill_shapes(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o,
                                                     lse, page_size)
    st = load().fa_paged_prefill_window(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                        block_table.data_ptr(), seq_lens.data_ptr(), cu_seqlens_q.data_ptr(),
                                        page_size, o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, num_pages,
                                        block_table.shape[1], int(max_q_len), 1 if causal else 0,
                                        int(window_left), int(window_right), float(scale), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_paged_prefill_window")