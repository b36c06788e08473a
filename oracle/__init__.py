"""CPU oracle for exact attention, in float64 -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The HIP library never calls it, and it shares no code, headers,
tables or helpers with the HIP path: its bf16 decoding, GQA head map, mask,
softmax, page gather and partial combine are all written out here again.

What it follows (pages cited by title and section):

* "FlashAttention et PagedAttention : a quoi servent-elles ?", section
  "FlashAttention : calculer sur le plan de travail": the attention equation
  softmax(Q K^T / sqrt(d_k)) V, whose softmax turns each score into a weight
  in [0, 1] that weights the values.
* "Flash Attention : pourquoi ton GPU utilise 85% de VRAM", section
  "L'attention classique en 3 etapes": the naive form in three materialised
  passes -- S = Q K^T of shape [batch, heads, seq, seq], P = softmax(S/sqrt d),
  O = P V of shape [batch, heads, seq, head_dim].  `attention_naive` is that
  form, written with the scale as an explicit argument.
* "FlashAttention" glossary page (polydesk.ai), section "L'idee cle :
  IO-awareness": the online softmax that carries the running max and running
  sum of exponentials over blocks and rescales to reach the exact result.
  `attention_online` is that recurrence; `combine_partials` applies the same
  rescaling across key partitions (split-K).
* "Variantes d'attention" (analyticslegends.ai), "Termes employes" (GQA):
  H_q query heads share H_kv < H_q K/V groups. Reading: contiguous groups,
  query head h uses K/V head h // (H_q / H_kv).
* "FlashAttention et PagedAttention ...", section "PagedAttention : ranger par
  pages plutot que d'un seul tenant": the KV cache is stored in fixed-size
  pages found through a lookup table, and no computation changes.
  `paged_decode` gathers the pages back into a contiguous cache and applies
  `attention_naive` to it.
* "FlashAttention" glossary page (polydesk.ai), section "FlashAttention vs
  PagedAttention": the two are complementary and used together (one computes
  attention, the other stores the KV cache). `paged_prefill` is that joint
  use for a chunk of new queries per sequence: gather the pages, then the
  attention equation with the causal mask.
* "Flash Attention : pourquoi ton GPU utilise 85% de VRAM", section "Ce que
  fait Flash Attention": the backward pass recomputes the attention matrix
  (block by block in the kernel) instead of storing it. `attention_backward`
  is the gradient of the attention equation written out by the chain rule
  on the fully materialised P -- the definition the recomputing kernel must
  reproduce.
* "FlashAttention" glossary page (polydesk.ai), section "FlashAttention-3":
  FP8 support with block quantization. `quantize_fp8` is block quantization
  to FP8 E4M3 (one float32 scale per block of rows, scale = block amax / 448,
  codes = E4M3 round-to-nearest-even of x / scale), `e4m3_encode` /
  `e4m3_decode` the format itself (1 sign, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals m * 2^-9, largest finite 448, no infinities,
  S.1111.111 = NaN), and `attention_fp8` the attention equation on the
  dequantized inputs (code value times its block's scale).
* Same section: FA3 pairs the block quantization with incoherent processing
  to limit the precision loss. Reading: Q and K rows are multiplied by one
  random orthogonal matrix before quantization, M = diag(s) H_d / sqrt(d)
  with s a vector of d random signs (drawn by the caller) and H_d Sylvester's
  Hadamard matrix. M M^T = I, so (Q M)(K M)^T = Q K^T and the attention is
  unchanged; an entry of unusual size is spread over all d channels. V is not
  transformed. `hadamard` is Sylvester's construction, `incoherent_transform`
  the product x diag(s) H_d / sqrt(d) written out, `quantize_fp8_incoherent`
  the transform followed by `quantize_fp8`.

Readings where the pages leave a step open:
* The scale is an explicit argument (the callers pass 1/sqrt(d) rounded to
  float32, promoted exactly to float64).
* Causal masking is bottom-right aligned: key j is visible from query i iff
  j <= i + (Nk - Nq). For Nq == Nk this is the usual lower triangle.
* LSE is the natural log of the sum over visible keys of exp(scale * q.k).
* A row with no visible key has O = 0 and LSE = -inf.
* Sliding window ("FlashAttention" glossary, section "FlashAttention et
  attention block-sparse": a block mask implements sliding windows): query
  at key position p sees keys p - left <= j <= p + right (-1: unbounded);
  causal forces right = 0.
* Block-sparse mask (same section: a mask over blocks of tokens says which
  blocks attend to each other): blocks are `block` = 128 consecutive query
  rows (i // block) and 128 consecutive keys (j // block), both counted from
  0; key j is visible from query i iff the mask entry of their block pair is
  nonzero, on top of the causal mask when causal is set. The mask may differ
  per batch and query head ([B, Hq, ceil(Nq/block), ceil(Nk/block)], numpy
  broadcasting allowed).
* Paged prefill: a sequence's n new queries are its last n tokens, so with
  the bottom-right causal mask query i of the chunk sees keys j <= i + (L - n)
  of its L cached tokens (which include the new tokens themselves).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "kv_head_of", "attention_naive", "attention_online",
    "combine_partials", "attention_split", "paged_decode", "gather_pages", "paged_prefill",
    "attention_backward", "e4m3_encode", "e4m3_decode", "quantize_fp8", "dequantize_fp8", "attention_fp8",
    "hadamard", "incoherent_transform", "quantize_fp8_incoherent",
]

_NEG_INF = -np.inf


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly: a bf16 value is the
    upper half of the float32 with the same sign, exponent and top mantissa
    bits, so shifting into the high half of a 32-bit word gives that float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    """float64 view of an input: uint16 arrays are bf16 bit patterns."""
    x = np.asarray(x)
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """GQA head map: contiguous groups of n_q_heads // n_kv_heads query heads."""
    if n_kv_heads <= 0 or n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a positive multiple of n_kv_heads")
    return h // (n_q_heads // n_kv_heads)


def _visible(i_rows: np.ndarray, n_q: int, n_k: int, causal: bool, window=None) -> np.ndarray:
    """Boolean [len(i_rows), n_k]: key j visible from query row i.

    Query i sits at key position p = i + (n_k - n_q) (bottom-right). causal
    keeps j <= p. window = (left, right), each -1 for unbounded, keeps
    p - left <= j <= p + right (a sliding window; causal forces right = 0).
    """
    j = np.arange(n_k)[None, :]
    p = i_rows[:, None] + (n_k - n_q)
    vis = np.ones((i_rows.size, n_k), dtype=bool)
    if causal:
        vis &= j <= p
    if window is not None:
        left, right = int(window[0]), int(window[1])
        if left >= 0:
            vis &= j >= p - left
        if right >= 0:
            vis &= j <= p + right
    return vis


def _block_visible(mask_bh: np.ndarray, i_rows: np.ndarray, n_k: int, block: int) -> np.ndarray:
    """Boolean [len(i_rows), n_k]: the block pair (i // block, j // block) is set."""
    qb = (i_rows // block)[:, None]
    kb = (np.arange(n_k) // block)[None, :]
    return mask_bh[qb, kb] != 0


def _rows_for(rows, b: int, h: int, n_q: int) -> np.ndarray:
    if rows is None:
        return np.arange(n_q)
    r = np.asarray(rows)
    if r.ndim == 1:
        return r.astype(np.int64)
    return r[b, h].astype(np.int64)


def attention_naive(q, k, v, scale: float, causal: bool, rows=None, return_p: bool = False,
                    row_block: int | None = None, window=None, block_mask=None, block: int = 128):
    """Three materialised passes per (batch, query head, block of query rows).

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] (float64).
    window: None, or (left, right) for a sliding window (see _visible).
    block_mask: None, or an array broadcastable to
    [B, Hq, ceil(Nq/block), ceil(Nk/block)]; nonzero = the block pair attends.
    rows: None (all rows), a 1-D array of query rows used for every (b, h), or
    an int array [B, Hq, R] of rows per head.
    Returns O [B, Hq, R, d] and LSE [B, Hq, R] (R = Nq when rows is None), and
    P [B, Hq, R, Nk] when return_p is set.

    Pass 1 writes S = scale * Q K^T with -inf at invisible keys; pass 2 reads S
    to write P = softmax(S) row-wise together with LSE = m + ln(sum exp(S - m));
    pass 3 reads P to write O = P V. Row blocks only bound the size of S.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = float(scale)
    R = Nq if rows is None else (np.asarray(rows).shape[-1])
    O = np.zeros((B, Hq, R, d))
    LSE = np.full((B, Hq, R), _NEG_INF)
    P_all = np.zeros((B, Hq, R, Nk)) if return_p else None
    if block_mask is not None:
        nqb, nkb = -(-Nq // block), -(-Nk // block)
        block_mask = np.broadcast_to(np.asarray(block_mask), (B, Hq, nqb, nkb))
    if row_block is None:
        row_block = max(1, min(1024, (1 << 22) // max(1, Nk)))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            Kg, Vg = k[b, g], v[b, g]
            r_idx = _rows_for(rows, b, h, Nq)
            for r0 in range(0, R, row_block):
                ii = r_idx[r0:r0 + row_block]
                # pass 1: scores
                S = s * (q[b, h, ii, :] @ Kg.T)
                vis = _visible(ii, Nq, Nk, causal, window)
                if block_mask is not None:
                    vis &= _block_visible(block_mask[b, h], ii, Nk, block)
                S = np.where(vis, S, _NEG_INF)
                # pass 2: softmax and log-sum-exp
                m = S.max(axis=1) if Nk else np.full(ii.size, _NEG_INF)
                ok = np.isfinite(m)
                E = np.zeros_like(S)
                E[ok] = np.exp(S[ok] - m[ok, None])
                l = E.sum(axis=1)
                P = np.zeros_like(S)
                P[ok] = E[ok] / l[ok, None]
                LSE[b, h, r0:r0 + ii.size] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), _NEG_INF)
                # pass 3: weighted sum of values
                O[b, h, r0:r0 + ii.size] = P @ Vg
                if return_p:
                    P_all[b, h, r0:r0 + ii.size] = P
    if return_p:
        return O, LSE, P_all
    return O, LSE


def attention_online(q, k, v, scale: float, causal: bool, tile: int, key_range=None):
    """Online softmax over key tiles of width `tile` (all in float64).

    Running state per query row: m (max so far, starts at -inf), l (sum of
    exp(S - m)), acc (sum of exp(S - m) * v). For each tile: m' = max(m, tile
    max); alpha = exp(m - m') (0 while m is -inf); l = alpha*l + sum exp(S - m');
    acc = alpha*acc + exp(S - m') V; m = m'. At the end O = acc / l and
    LSE = m + ln l. `key_range` = (j0, j1) restricts the keys swept (used for
    split-K partials); masking always uses the global key index.
    Returns O [B, Hq, Nq, d], LSE [B, Hq, Nq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    j_lo, j_hi = (0, Nk) if key_range is None else key_range
    if tile < 1:
        raise ValueError("tile must be >= 1")
    s = float(scale)
    O = np.zeros((B, Hq, Nq, d))
    LSE = np.full((B, Hq, Nq), _NEG_INF)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            m = np.full(Nq, _NEG_INF)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, d))
            for j0 in range(j_lo, j_hi, tile):
                j1 = min(j0 + tile, j_hi)
                S = s * (q[b, h] @ k[b, g, j0:j1].T)
                vis = _visible(rows, Nq, Nk, causal)[:, j0:j1]
                S = np.where(vis, S, _NEG_INF)
                m_new = np.maximum(m, S.max(axis=1))
                alpha = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - np.where(np.isfinite(m_new), m_new, 0.0)), 0.0)
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                Pt = np.where(vis, np.exp(S - ref[:, None]), 0.0)
                l = alpha * l + Pt.sum(axis=1)
                acc = alpha[:, None] * acc + Pt @ v[b, g, j0:j1]
                m = m_new
            ok = l > 0
            O[b, h] = np.where(ok[:, None], acc / np.where(ok, l, 1.0)[:, None], 0.0)
            LSE[b, h] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), _NEG_INF)
    return O, LSE


def combine_partials(o_parts, lse_parts):
    """Merge per-partition results (O_s normalised, LSE_s) over axis 0.

    LSE = M + ln sum_s exp(LSE_s - M) with M = max_s LSE_s, and
    O = sum_s exp(LSE_s - LSE) O_s. Partitions with LSE_s = -inf (no visible
    key) carry zero weight; if all are empty, O = 0 and LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    ok = np.isfinite(M)
    Mz = np.where(ok, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Mz[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(ok, Mz + np.log(np.where(ok, tot, 1.0)), _NEG_INF)
    lz = np.where(ok, lse, 0.0)
    wn = np.where(np.isfinite(lse_parts), np.exp(lse_parts - lz[None]), 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    o = np.where(ok[..., None], o, 0.0)
    return o, lse


def attention_split(q, k, v, scale: float, causal: bool, bounds, tile: int = 16):
    """Split-K: run the online recurrence on each contiguous key range
    [bounds[i], bounds[i+1]) (ranges may be empty) and merge the partials."""
    parts = [attention_online(q, k, v, scale, causal, tile, (bounds[i], bounds[i + 1]))
             for i in range(len(bounds) - 1)]
    return combine_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


def gather_pages(pool, block_table_row, seq_len: int, page_size: int) -> np.ndarray:
    """Contiguous cache [H_kv, L, d] of one sequence from a paged pool
    [num_pages, H_kv, page_size, d]: token t lives in page
    block_table_row[t // page_size] at slot t % page_size."""
    t = np.arange(seq_len)
    pages = np.asarray(block_table_row)[t // page_size].astype(np.int64)
    slots = t % page_size
    g = np.asarray(pool)[pages, :, slots, :]          # [L, H_kv, d]
    return np.ascontiguousarray(np.transpose(g, (1, 0, 2)))


def paged_decode(q, k_pool, v_pool, block_table, seq_lens, scale: float, page_size: int = 16):
    """One new query token per sequence against its paged KV cache.

    q: [B, Hq, d]; pools: [num_pages, Hkv, page_size, d], float or bf16 bit
    patterns (uint16, decoded after the gather); block_table
    [B, max_pages] (entries past the sequence's pages are never read);
    seq_lens [B]. The query sees every cached token (no mask).
    Returns O [B, Hq, d], LSE [B, Hq].
    """
    q = _as_f64(q)
    B, Hq, d = q.shape
    O = np.zeros((B, Hq, d))
    LSE = np.full((B, Hq), _NEG_INF)
    for b in range(B):
        L = int(seq_lens[b])
        kb = _as_f64(gather_pages(k_pool, block_table[b], L, page_size))
        vb = _as_f64(gather_pages(v_pool, block_table[b], L, page_size))
        o, lse = attention_naive(q[b][None, :, None, :], kb[None], vb[None], scale, causal=False)
        O[b] = o[0, :, 0, :]
        LSE[b] = lse[0, :, 0]
    return O, LSE


def paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, scale: float, causal: bool,
                  page_size: int = 16, window=None):
    """A chunk of new queries per sequence against its paged KV cache.

    q: [total_q, Hq, d] packed rows; sequence b owns rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1, its last n_b tokens. pools:
    [num_pages, Hkv, page_size, d] (float or bf16 bit patterns);
    block_table [B, max_pages]; seq_lens [B] (cached tokens L_b, the new
    ones included). Each sequence's cache is gathered (gather_pages) and
    `attention_naive` runs on it with Nq = n_b, Nk = L_b, so the causal mask
    is the bottom-right one (and so is a sliding window, window = (left,
    right) as for attention_naive). Returns O [total_q, Hq, d], LSE
    [total_q, Hq].
    """
    q = _as_f64(q)
    total_q, Hq, d = q.shape
    O = np.zeros((total_q, Hq, d))
    LSE = np.full((total_q, Hq), _NEG_INF)
    for b in range(len(seq_lens)):
        c0, c1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        if c1 == c0:
            continue
        L = int(seq_lens[b])
        kb = _as_f64(gather_pages(k_pool, block_table[b], L, page_size))
        vb = _as_f64(gather_pages(v_pool, block_table[b], L, page_size))
        qb = np.transpose(q[c0:c1], (1, 0, 2))[None]          # [1, Hq, n_b, d]
        o, lse = attention_naive(qb, kb[None], vb[None], scale, causal, window=window)
        O[c0:c1] = np.transpose(o[0], (1, 0, 2))
        LSE[c0:c1] = lse[0].T
    return O, LSE


def attention_backward(q, k, v, do, scale: float, causal: bool, window=None, block_mask=None, block: int = 128):
    """Gradients of O = softmax(scale * Q K^T + mask) V for an incoming dO.

    q, do: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] (float64). Per (batch,
    query head h, K/V head g = h // (Hq / Hkv)), with P the row softmax of the
    masked scores (as in attention_naive; rows with no visible key have P = 0):
        dP = dO V^T
        dS = P * (dP - rowsum(dP * P))       the softmax Jacobian, row by row
        dQ = scale * dS K
        dK_g += scale * dS^T Q,   dV_g += P^T dO   (summed over the group's heads)
    Returns dq [B, Hq, Nq, d], dk [B, Hkv, Nk, d], dv [B, Hkv, Nk, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = float(scale)
    if block_mask is not None:
        block_mask = np.broadcast_to(np.asarray(block_mask), (B, Hq, -(-Nq // block), -(-Nk // block)))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(Nq)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            Kg, Vg = k[b, g], v[b, g]
            vis = _visible(rows, Nq, Nk, causal, window)
            if block_mask is not None:
                vis &= _block_visible(block_mask[b, h], rows, Nk, block)
            S = np.where(vis, s * (q[b, h] @ Kg.T), _NEG_INF)
            m = S.max(axis=1) if Nk else np.full(Nq, _NEG_INF)
            ok = np.isfinite(m)
            E = np.zeros_like(S)
            E[ok] = np.exp(S[ok] - m[ok, None])
            P = np.zeros_like(S)
            P[ok] = E[ok] / E[ok].sum(axis=1, keepdims=True)
            dP = do[b, h] @ Vg.T
            dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
            dq[b, h] = s * (dS @ Kg)
            dk[b, g] += s * (dS.T @ q[b, h])
            dv[b, g] += P.T @ do[b, h]
    return dq, dk, dv


def e4m3_decode(codes) -> np.ndarray:
    """FP8 E4M3 codes (uint8) to their float64 values."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Round float values to FP8 E4M3 codes: round to nearest, ties to even
    mantissa; magnitudes past 448 saturate to 448 (the quantizer below never
    produces them beyond rounding)."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.int64) << 7
    a = np.minimum(np.abs(x), 448.0)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6                      # below the smallest normal: m * 2^-9, m = 0..8
    ms = np.rint(a * 2.0 ** 9)               # exact scaling; rint = ties to even
    out = np.where(sub, ms.astype(np.int64), out)   # m = 8 is code 8 = 2^-6, the smallest normal
    e = np.floor(np.log2(np.where(sub, 1.0, a)))
    mant = np.rint((np.where(sub, 1.0, a) / np.exp2(e) - 1.0) * 8.0)  # (a / 2^e - 1) * 8 is exact
    carry = mant == 8.0
    e = e + carry
    mant = np.where(carry, 0.0, mant)
    normal = ((e.astype(np.int64) + 7) << 3) | mant.astype(np.int64)
    out = np.where(sub, out, normal)
    return (out | sign).astype(np.uint8)


def quantize_fp8(x, block_rows: int):
    """Block quantization of x [B, H, N, d] (float values that float32 holds
    exactly, e.g. bf16 inputs) to E4M3: rows [block_rows*i, block_rows*(i+1))
    of each (b, h) share one float32 scale = amax / 448 (1 for an all-zero
    block), computed and applied in float32: codes = E4M3(x / scale).
    Returns codes uint8 [B, H, N, d] and scales float32 [B, H, ceil(N / block_rows)]."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = -(-N // block_rows)
    scales = np.ones((B, H, nb), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for i in range(nb):
        blk = x[:, :, i * block_rows:(i + 1) * block_rows]
        amax = np.abs(blk).max(axis=(2, 3)) if blk.size else np.zeros((B, H), np.float32)
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        scales[:, :, i] = sc
        q = (blk / sc[:, :, None, None]).astype(np.float32)   # float32 division, correctly rounded
        codes[:, :, i * block_rows:(i + 1) * block_rows] = e4m3_encode(q)
    return codes, scales


def dequantize_fp8(codes, scales, block_rows: int) -> np.ndarray:
    """Code values times their block's scale, float64 [B, H, N, d]."""
    v = e4m3_decode(codes)
    N = v.shape[2]
    rows = np.arange(N) // block_rows
    return v * np.asarray(scales, dtype=np.float64)[:, :, rows][..., None]


def attention_fp8(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, scale: float, causal: bool,
                  q_block: int = 128, k_block: int = 128, v_block=None, rows=None):
    """The attention equation (attention_naive) on the dequantized FP8 inputs.
    v_block None: one V scale per (batch, head) (v_scales [B, Hkv, 1])."""
    q = dequantize_fp8(q_codes, q_scales, q_block)
    k = dequantize_fp8(k_codes, k_scales, k_block)
    v = dequantize_fp8(v_codes, v_scales, v_block if v_block is not None else max(1, np.asarray(v_codes).shape[2]))
    return attention_naive(q, k, v, scale, causal, rows=rows)


def hadamard(d: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order d (a power of two), float64:
    H_1 = [1] and H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def incoherent_transform(x, signs) -> np.ndarray:
    """Rows of x [..., d] times M = diag(signs) H_d / sqrt(d), float64: each
    channel i is first multiplied by signs[i] (+1 or -1), then the row by the
    Hadamard matrix, then by 1 / sqrt(d). M is orthogonal."""
    x = _as_f64(x)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float64).reshape(d)
    if not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be +1 or -1")
    m = (s[:, None] * hadamard(d)) / np.sqrt(d)
    return x @ m


def quantize_fp8_incoherent(x, signs, block_rows: int):
    """Incoherent processing, then block quantization: y =
    incoherent_transform(x, signs) in float64, rounded once to float32, then
    quantize_fp8(y, block_rows) (scale = block amax / 448, codes = E4M3 of
    y / scale, both in float32). Returns codes uint8 [B, H, N, d] and scales
    float32 [B, H, ceil(N / block_rows)]; the dequantized values approximate
    x M, so Q and K quantized this way with the same signs give Q K^T."""
    y = incoherent_transform(x, signs).astype(np.float32)
    return quantize_fp8(y, block_rows)
