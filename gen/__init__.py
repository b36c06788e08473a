"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path.

This module holds none of the attention arithmetic: it only produces bytes
(bf16 bit patterns, int32 tables) from a (seed, stream, index) counter, so that
both sides of every parity check consume identical inputs. The generator itself
(SplitMix64 + Box-Muller + bf16 round-to-nearest-even) is defined in gen.c.

Stream numbers used throughout the tests and the bench:
  0 = Q (or the decode query), 1 = K (or the K pool), 2 = V (or the V pool),
  3 = sequence lengths, 4 = page permutation, 5 = sampled query rows,
  6 = block-sparse mask entries, 7 = the backward's incoming gradient dO,
  8 = which entries of an outlier input are enlarged, 9 = random signs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_SEQLENS, STREAM_PERM, STREAM_ROWS, STREAM_MASK, STREAM_DO, STREAM_OUTLIER, STREAM_SIGNS = range(10)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libgen.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile gen.c into libgen.so next to it (gcc, OpenMP)."""
    src = os.path.join(_HERE, "gen.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def build_host_sanitized(out_dir: str) -> str:
    """libgen_hostsan.so in out_dir: gen.c under gcc's AddressSanitizer and
    UndefinedBehaviorSanitizer (loaded by tests/test_host_sanitizers.py)."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libgen_hostsan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", os.path.join(_HERE, "gen.c"), "-o", out, "-lm"])
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
        vp = ctypes.c_void_p
        lib.gen_stream_key.argtypes = [u64, u64]
        lib.gen_stream_key.restype = u64
        lib.gen_draw.argtypes = [u64, u64, u64]
        lib.gen_draw.restype = u64
        lib.gen_normal_bf16.argtypes = [u64, u64, f32, u64, u64, vp]
        lib.gen_normal_bf16.restype = None
        lib.gen_normal_f32.argtypes = [u64, u64, f32, u64, u64, vp]
        lib.gen_normal_f32.restype = None
        lib.gen_uniform_int.argtypes = [u64, u64, i64, i64, u64, u64, vp]
        lib.gen_uniform_int.restype = None
        lib.gen_permutation.argtypes = [u64, u64, u64, vp]
        lib.gen_permutation.restype = None
        _lib = lib
    return _lib


def draw(seed: int, stream: int, index: int) -> int:
    """Raw 64-bit draw `index` of `stream` under `seed`."""
    return int(_load().gen_draw(seed, stream, index))


def normal_bf16(seed: int, stream: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of sigma * N(0,1), elements offset.. of the stream."""
    out = np.empty(shape, dtype=np.uint16)
    if out.size:
        _load().gen_normal_bf16(seed, stream, sigma, offset, out.size, out.ctypes.data)
    return out


def normal_f32(seed: int, stream: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    """The same sequence before the bf16 narrowing."""
    out = np.empty(shape, dtype=np.float32)
    if out.size:
        _load().gen_normal_f32(seed, stream, sigma, offset, out.size, out.ctypes.data)
    return out


def outlier_bf16(seed: int, stream: int, shape, per_million: int = 1000, factor: float = 16.0) -> np.ndarray:
    """bf16 bit patterns of N(0,1) (normal_bf16 of `stream`) in which each
    entry, with probability per_million / 10^6, is multiplied by `factor`, a
    power of two (so the product is still a bf16 value). Entry e is enlarged
    iff draw e of stream 8, sub-sequence `stream`, uniform on [0, 10^6 - 1],
    is below per_million."""
    if factor <= 0 or np.log2(factor) != np.round(np.log2(factor)):
        raise ValueError("factor must be a power of two")
    bits = normal_bf16(seed, stream, shape)
    n = bits.size
    pick = uniform_int(seed, STREAM_OUTLIER, n, 0, 999999, offset=int(stream) << 40) < per_million
    x = (bits.astype(np.uint32) << 16).view(np.float32).reshape(-1)
    x = np.where(pick, x * np.float32(factor), x).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16).reshape(shape)


def random_signs(seed: int, n: int) -> np.ndarray:
    """n signs, -1 or +1, as int8: entry e is -1 iff draw e of stream 9,
    uniform on [0, 1], is 1."""
    return (1 - 2 * uniform_int(seed, STREAM_SIGNS, n, 0, 1)).astype(np.int8)


def uniform_int(seed: int, stream: int, n: int, lo: int, hi: int, offset: int = 0) -> np.ndarray:
    """n integers uniform on [lo, hi] (inclusive), as int64."""
    if lo > hi:
        raise ValueError("lo > hi")
    out = np.empty(n, dtype=np.int64)
    if n:
        _load().gen_uniform_int(seed, stream, lo, hi, offset, n, out.ctypes.data)
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """Seeded permutation of [0, n) (Durstenfeld's Fisher-Yates), as int64."""
    out = np.empty(n, dtype=np.int64)
    if n:
        _load().gen_permutation(seed, stream, n, out.ctypes.data)
    return out


def decode_layout(seed: int, batch: int, len_lo: int, len_hi: int, page_size: int = 16,
                  max_pages_per_seq: int | None = None, seq_lens=None):
    """Sequence lengths and a paged block table for a decode batch.

    Lengths are uniform integers on [len_lo, len_hi] (stream 3) unless given.
    Sequence b owns ceil(L_b / page_size) logical pages; the physical page ids
    are a seeded permutation (stream 4) of [0, total_pages) dealt out in order
    b = 0, 1, ... and logical page 0, 1, ... . Unused table entries are -1.

    Returns (seq_lens int32 [B], block_table int32 [B, max_pages_per_seq],
    total_pages).
    """
    if seq_lens is None:
        seq_lens = uniform_int(seed, STREAM_SEQLENS, batch, len_lo, len_hi)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    npages = (seq_lens + page_size - 1) // page_size
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, -(-len_hi // page_size))
    if npages.size and int(npages.max()) > max_pages_per_seq:
        raise ValueError("a sequence needs more pages than max_pages_per_seq")
    total = int(npages.sum())
    perm = permutation(seed, STREAM_PERM, total)
    table = np.full((batch, max_pages_per_seq), -1, dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(npages)[:-1]]) if batch else np.zeros(0, np.int64)
    for b in range(batch):
        n = int(npages[b])
        table[b, :n] = perm[starts[b]:starts[b] + n]
    return seq_lens.astype(np.int32), table, total


def random_block_mask(seed: int, shape, percent: int) -> np.ndarray:
    """uint8 mask of the given shape whose entries are 1 with probability
    percent/100: entry e is 1 iff draw e of stream 6 (uniform on [0, 99]) is
    below percent."""
    n = int(np.prod(shape))
    u = uniform_int(seed, STREAM_MASK, n, 0, 99)
    return (u < percent).astype(np.uint8).reshape(shape)


def local_global_block_mask(n_qblocks: int, n_kblocks: int, local: int, n_global: int) -> np.ndarray:
    """uint8 [n_qblocks, n_kblocks]: query block qb attends to the first
    n_global key blocks and to the `local` key blocks ending at its own
    position (kb in [qb - local + 1, qb]); no randomness."""
    qb = np.arange(n_qblocks)[:, None]
    kb = np.arange(n_kblocks)[None, :]
    return ((kb < n_global) | ((kb <= qb) & (kb > qb - local))).astype(np.uint8)


def row_sample(seed: int, n_rows: int, count: int, salt: int = 0) -> np.ndarray:
    """Sorted distinct query rows: 0, n_rows-1 and count-2 more drawn by a
    partial Fisher-Yates shuffle of [1, n_rows-2] (stream 5; `salt` selects an
    independent sub-sequence, e.g. one per head)."""
    if count >= n_rows:
        return np.arange(n_rows, dtype=np.int64)
    pool = np.arange(1, n_rows - 1, dtype=np.int64)
    k = count - 2
    base = int(salt) << 32
    for s in range(k):
        j = s + draw(seed, STREAM_ROWS, base + s) % (pool.size - s)
        pool[s], pool[j] = pool[j], pool[s]
    return np.sort(np.concatenate([[0, n_rows - 1], pool[:k]])).astype(np.int64)
