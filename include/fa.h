/*
 * fa.h -- exact attention forward for AMD MI355X (gfx950), C ABI.
 *
 * Computes O = softmax(scale * Q K^T + mask) V tile by tile with an online
 * softmax, so the score matrix never reaches device memory, and returns the
 * per-row log-sum-exp (LSE) beside O.
 *
 * Sources of the operations (page title, section):
 *   - the attention equation and its softmax weights: "FlashAttention et
 *     PagedAttention : a quoi servent-elles ?", section "FlashAttention :
 *     calculer sur le plan de travail";
 *   - tiling and the online softmax (running max and running sum of
 *     exponentials, rescaled per block, exact result): "FlashAttention"
 *     glossary (polydesk.ai), section "L'idee cle : IO-awareness"; and
 *     "Comment Flash Attention reduit-il le trafic memoire ...", sections on
 *     tiles and on the online softmax;
 *   - shapes [batch, heads, seq_len, head_dim]: "Flash Attention : pourquoi
 *     ton GPU utilise 85% de VRAM", section "L'attention classique en 3
 *     etapes";
 *   - GQA (H_q query heads sharing H_kv K/V heads): "Variantes d'attention",
 *     "Termes employes sur cette page";
 *   - the paged KV cache (fixed-size pages found through a lookup table, with
 *     the computation unchanged): "FlashAttention et PagedAttention ...",
 *     section "PagedAttention : ranger par pages plutot que d'un seul tenant".
 *
 * Conventions shared by every entry point:
 *   - Element types: Q, K, V, O are bfloat16 (passed as void*); LSE is float.
 *   - All tensors are dense and row-major (last index fastest), in device
 *     memory owned by the caller. The library never allocates, frees or
 *     synchronises; it only enqueues kernels on `stream` (a hipStream_t;
 *     NULL means the null stream) and returns.
 *   - GQA head map: query head h reads K/V head h / (Hq / Hkv) (contiguous
 *     groups). Hq must be a multiple of Hkv; Hkv == Hq is MHA, Hkv == 1 MQA.
 *   - LSE[row] = ln sum over visible keys j of exp(scale * q_row . k_j).
 *     A row with no visible key gets O = 0 and LSE = -infinity.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call returns a negative fa_status and enqueues nothing. Unsupported
 *     input is reported, never routed to another implementation.
 *   - Values that live in device memory (block_table, seq_lens) cannot be
 *     checked without a synchronisation and are not checked: the caller
 *     guarantees the ranges stated below.
 *   - No global mutable state, except the allocation-free decode's
 *     per-device scratch (fa_paged_decode_noalloc): calls are thread-safe;
 *     calls on one stream run in order.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,     /* a size is out of range (negative, zero where not allowed, too large) */
    FA_ERR_GQA = -3,       /* Hq is not a positive multiple of Hkv */
    FA_ERR_HEADDIM = -4,   /* head dimension not supported (64 and 128 are) */
    FA_ERR_PAGESIZE = -5,  /* page size not supported (16 is) */
    FA_ERR_WORKSPACE = -6, /* workspace NULL or too small (allocation-free decode: sizes past its scratch) */
    FA_ERR_SCALE = -7,     /* scale is not finite and positive */
    FA_ERR_WINDOW = -8,    /* a window bound is below -1 */
    FA_ERR_HIP = -100      /* the HIP runtime reported an error while enqueuing */
} fa_status;

/*
 * Prefill / full attention forward.
 *
 *   q   [B, Hq,  Nq, d]  bf16       k, v [B, Hkv, Nk, d]  bf16
 *   o   [B, Hq,  Nq, d]  bf16 (out) lse  [B, Hq,  Nq]     float (out)
 *
 * causal != 0 masks key j from query i unless j <= i + (Nk - Nq) (the causal
 * diagonal aligned to the last query and last key; for Nq == Nk it is the
 * lower triangle, j <= i). causal == 0 lets every query see every key.
 * scale multiplies Q K^T before the softmax (1/sqrt(d) for the standard
 * attention equation); it must be finite and > 0.
 *
 * Sizes: B, Hq, Hkv >= 1; Nq, Nk >= 0 (Nq == 0 is a no-op that returns FA_OK;
 * Nk == 0 gives O = 0 and LSE = -inf for every row); d in {64, 128};
 * every tensor holds fewer than 2^40 elements and Nq, Nk < 2^30.
 * Pointers: q, o, lse are required when Nq > 0; k, v when Nk > 0.
 * o and lse must not overlap the inputs.
 * Returns FA_OK once the kernel is enqueued, or a negative fa_status.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               int causal, float scale, void* stream);

/*
 * Prefill / full attention forward with a sliding window (local attention).
 * Source: "FlashAttention" glossary (polydesk.ai), section "FlashAttention et
 * attention block-sparse": a mask of which token blocks attend to each
 * other implements sliding windows while the computation stays tiled; and
 * "FlashAttention et PagedAttention : à quoi servent-elles ?" (ranksignal.fr),
 * section "Trois idées reçues à écarter": a sliding window looks only at the
 * most recent tokens (window_left = w - 1 with causal: the last w tokens).
 *
 * Same tensors, sizes and errors as fa_forward, plus two bounds. Query i sits
 * at key position p = i + (Nk - Nq) (bottom-right, as for the causal mask)
 * and sees key j iff
 *     (window_left  < 0 or j >= p - window_left) and
 *     (window_right < 0 or j <= p + window_right) and
 *     (causal == 0 or j <= p).
 * -1 means unbounded; causal != 0 forces the right bound to 0. Key tiles
 * wholly outside every row's window of a workgroup are never read.
 * Rows with no visible key get O = 0 and LSE = -inf.
 * Returns FA_ERR_WINDOW for a bound below -1; otherwise as fa_forward.
 */
int fa_forward_window(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      int causal, int window_left, int window_right, float scale, void* stream);

/* Queries and keys per block of a block-sparse mask, and the most key blocks
 * (so Nk <= FA_SPARSE_MAX_KEY_BLOCKS * FA_SPARSE_BLOCK) it supports. */
#define FA_SPARSE_BLOCK 128
#define FA_SPARSE_MAX_KEY_BLOCKS 4096

/*
 * Prefill / full attention forward with a block-sparse mask.
 * Source: "FlashAttention" glossary (polydesk.ai), section "FlashAttention et
 * attention block-sparse": instead of every token pair, a mask over blocks
 * of tokens says which blocks attend to each other (local + global
 * patterns, document masks), and the computation keeps its tiling and
 * online softmax.
 *
 * Same tensors, sizes and errors as fa_forward, plus the mask:
 *   block_mask  bytes, entry (b, h, qb, kb) at
 *               block_mask[b * mask_stride_b + h * mask_stride_h + qb * KB + kb]
 *               for query head h, query block qb < ceil(Nq / 128) and key
 *               block kb < KB = ceil(Nk / 128); nonzero = the block pair
 *               attends. Strides are in bytes (elements), >= 0; 0 broadcasts
 *               one mask over batches or heads. Read only, owned by the caller.
 * Query i is in block i / 128 and key j in block j / 128 (both counted from
 * 0). Key j is visible from query i iff their block pair is set and, when
 * causal != 0, j <= i + (Nk - Nq). Key blocks that no row of a workgroup's
 * row blocks uses are never read. Rows with no visible key get O = 0 and
 * LSE = -inf.
 * Returns FA_ERR_SHAPE if ceil(Nk / 128) > FA_SPARSE_MAX_KEY_BLOCKS or a
 * stride is negative, FA_ERR_NULL if block_mask is NULL (Nq > 0); otherwise
 * as fa_forward.
 */
int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            const uint8_t* block_mask, long long mask_stride_b, long long mask_stride_h,
                            float scale, void* stream);

/* Rows per Q / K scale block of the FP8 forward. */
#define FA_FP8_SCALE_ROWS 128

/*
 * Block quantization to FP8 E4M3 (the OCP format: 1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, largest finite 448, no infinities).
 * Source: "FlashAttention" glossary (polydesk.ai), section
 * "FlashAttention-3": FP8 support with block quantization.
 *
 *   x       [B, H, N, d]                    bf16 (in)
 *   codes   [B, H, N, d]                    uint8 E4M3 (out)
 *   scales  [B, H, ceil(N / block_rows)]    float (out)
 *
 * Rows [block_rows * i, block_rows * (i + 1)) of each (b, h) form a block
 * with scale = (largest |x| in the block) / 448 (1 for an all-zero block);
 * codes = E4M3(x / scale), round-to-nearest-even, both in float32. So the
 * block's largest element maps to +-448. Use block_rows = 128
 * (FA_FP8_SCALE_ROWS) for Q and K and block_rows = N for V (one scale per
 * head) to feed fa_forward_fp8. d in {64, 128}. N == 0 is a no-op.
 */
int fa_quantize_fp8(const void* x, uint8_t* codes, float* scales, int B, int H, int N, int d, int block_rows,
                    void* stream);

/*
 * Incoherent processing fused with the block quantization above.
 * Source: "FlashAttention" glossary (polydesk.ai), section
 * "FlashAttention-3": FP8 with block quantization and incoherent processing
 * to limit the precision loss.
 *
 *   x       [B, H, N, d]                    bf16 (in)
 *   signs   [d]                             int8 (in): channel i is negated
 *                                           where signs[i] < 0
 *   codes   [B, H, N, d]                    uint8 E4M3 (out)
 *   scales  [B, H, ceil(N / block_rows)]    float (out)
 *
 * Each row x is replaced by y = x diag(s) H_d / sqrt(d), with s_i = -1 where
 * signs[i] < 0 and +1 otherwise, and H_d Sylvester's Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)); y is computed in float32. Then y is
 * quantized exactly as fa_quantize_fp8 quantizes x. The matrix is orthogonal:
 * Q and K quantized with the same signs (drawn at random by the caller, one
 * vector for all heads) give fa_forward_fp8 the scores of the original Q K^T,
 * while a large entry of a row is spread over all d channels before it sets
 * its block's scale. V is quantized with fa_quantize_fp8 (not transformed).
 * d in {64, 128}; x, codes 16-byte aligned (as fa_quantize_fp8).
 * N == 0 is a no-op. Errors as fa_quantize_fp8 (FA_ERR_NULL for signs too).
 */
int fa_quantize_fp8_incoherent(const void* x, const int8_t* signs, uint8_t* codes, float* scales, int B, int H,
                               int N, int d, int block_rows, void* stream);

/*
 * Attention forward on FP8 E4M3 inputs with block scales.
 * Source: "FlashAttention" glossary (polydesk.ai), section
 * "FlashAttention-3": FP8 with block quantization.
 *
 *   q         [B, Hq, Nq, d]  E4M3 codes   q_scales  [B, Hq, ceil(Nq / 128)] float
 *   k         [B, Hkv, Nk, d] E4M3 codes   k_scales  [B, Hkv, ceil(Nk / 128)] float
 *   v         [B, Hkv, Nk, d] E4M3 codes   v_scales  [B, Hkv] float
 *   o         [B, Hq, Nq, d]  bf16 (out)   lse       [B, Hq, Nq] float (out)
 *
 * Computes fa_forward's result for the dequantized inputs (code value times
 * its block's scale): Q rows [128 i, 128 i + 128) of a head use q_scales[.., i],
 * K rows likewise, V one scale per (batch, K/V head). The probabilities are
 * rounded to E4M3 for the P V product (values up to 2^8, relative step 2^-3),
 * so O carries that rounding on top of fa_forward's. causal, scale, sizes and
 * errors as fa_forward (plus FA_ERR_NULL for a missing scale array).
 */
int fa_forward_fp8(const uint8_t* q, const float* q_scales, const uint8_t* k, const float* k_scales,
                   const uint8_t* v, const float* v_scales, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, int causal, float scale, void* stream);

/*
 * Bytes of device workspace fa_backward needs: two floats per query row
 * (B * Hq * Nq * 8: the row sums rowsum(dO * O), then the LSE in base-2
 * units). Returns 0 for invalid sizes.
 */
size_t fa_backward_workspace_size(int B, int Hq, int Nq);

/*
 * Attention backward: the gradients dQ, dK, dV of the forward's
 * O = softmax(scale * Q K^T + mask) V for an incoming gradient dO.
 * Source: "Flash Attention : pourquoi ton GPU utilise 85% de VRAM"
 * (patricehuetz.fr), section "Ce que fait Flash Attention": the backward
 * recomputes the attention matrix block by block instead of storing it. Here
 * P = exp(scale * Q K^T - LSE) is recomputed tile by tile from the forward's
 * LSE, with dS = P * (dO V^T - rowsum(dO * O)), dQ = scale dS K,
 * dK = scale dS^T Q, dV = P^T dO (dK and dV summed over the query heads that
 * share a K/V head). Nothing of size Nq x Nk is written.
 *
 *   q, o, dout, dq  [B, Hq,  Nq, d]  bf16 (dq out)
 *   k, v, dk, dv    [B, Hkv, Nk, d]  bf16 (dk, dv out)
 *   lse             [B, Hq,  Nq]     float, as fa_forward wrote it for (q, k, v)
 *   workspace       >= fa_backward_workspace_size(B, Hq, Nq) bytes of device
 *                   memory (per-row values; contents on entry are ignored)
 *
 * causal, scale and the size limits are those of fa_forward (o and lse must
 * be the forward's outputs for the same causal flag and scale). Rows with no
 * visible key get dq = 0 and contribute nothing to dk and dv. The result is
 * deterministic (no atomics). Outputs must not overlap inputs or each other.
 * Returns FA_ERR_NULL for a missing pointer, FA_ERR_WORKSPACE for a missing
 * or small workspace (Nq > 0), otherwise as fa_forward.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the sliding-window forward (fa_forward_window): the gradients
 * of O = softmax(scale * Q K^T + mask) V where the mask keeps, for query i
 * at key position p = i + Nk - Nq, the keys p - window_left <= j <= p +
 * window_right (-1 for an unbounded side; causal forces the right bound to
 * 0). Sources: the window as for fa_forward_window ("FlashAttention" glossary,
 * section "FlashAttention et attention block-sparse"; "FlashAttention et
 * PagedAttention : à quoi servent-elles ?", section "Trois idées reçues à
 * écarter"), the recomputation as for fa_backward ("Flash Attention : pourquoi
 * ton GPU utilise 85% de VRAM", section "Ce que fait Flash Attention").
 * Tensors, workspace, determinism and status codes as for
 * fa_backward, plus FA_ERR_WINDOW for a bound below -1; o and lse must come
 * from fa_forward_window with the same window, causal flag and scale.
 */
int fa_backward_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       int causal, int window_left, int window_right, float scale, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The block-sparse backward's limit on (Hq / Hkv) * ceil(Nq / 64), the
 * steps of one key block's dK/dV work. */
#define FA_SPARSE_MAX_BACKWARD_STEPS 131072

/*
 * Bytes of device workspace fa_backward_block_sparse needs: fa_backward's
 * (two floats per query row) and, when one key block's share of the dK/dV
 * work may be long enough to be split over several workgroups, fp32 partial
 * dK and dV for each piece (at most about 16 * Nk * d * 8 bytes beyond the
 * per-row values). Returns 0 for invalid sizes (including
 * (Hq / Hkv) * ceil(Nq / 64) > FA_SPARSE_MAX_BACKWARD_STEPS) or B == 0.
 */
size_t fa_backward_block_sparse_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * Backward of the block-sparse forward (fa_forward_block_sparse): the
 * gradients of O = softmax(scale * Q K^T + mask) V where key j is visible
 * from query i iff their 128 x 128 block pair is set in block_mask (and,
 * when causal != 0, j <= i + Nk - Nq). Sources: the mask as for
 * fa_forward_block_sparse ("FlashAttention" glossary, section
 * "FlashAttention et attention block-sparse": block masks in the forward
 * and in the backward pass), the recomputation as for fa_backward
 * ("Flash Attention : pourquoi ton GPU
 * utilise 85% de VRAM", section "Ce que fait Flash Attention").
 * block_mask, its strides and their limits as for fa_forward_block_sparse,
 * plus (Hq / Hkv) * ceil(Nq / 64) <= FA_SPARSE_MAX_BACKWARD_STEPS
 * (FA_ERR_SHAPE otherwise); tensors, determinism and the other status codes
 * as for fa_backward; the
 * workspace must hold fa_backward_block_sparse_workspace_size(B, Hq, Hkv,
 * Nq, Nk, d) bytes (contents on entry are ignored). o and lse must come from
 * fa_forward_block_sparse with the same mask, causal flag and scale. Block pairs the mask clears are never
 * read: a query block's rows of dQ only gather its visible key blocks, a
 * key block's dK, dV only its visible (query block, head) pairs; keys that
 * no query sees get dk = dv = 0.
 */
int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, const uint8_t* block_mask, long long mask_stride_b,
                             long long mask_stride_h, float scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Bytes of device workspace fa_paged_decode needs for these sizes (the
 * split-K partial outputs and partial LSEs). Returns 0 for invalid sizes.
 * The value is monotone non-decreasing in every argument.
 */
size_t fa_paged_decode_workspace_size(int B, int Hq, int d, int page_size, int max_seq_len);

/*
 * Decode attention over a paged KV cache: one new query token per sequence.
 *
 *   q           [B, Hq, d]                          bf16
 *   k_pool      [num_pages, Hkv, page_size, d]      bf16
 *   v_pool      [num_pages, Hkv, page_size, d]      bf16
 *   block_table [B, max_pages_per_seq]              int32
 *   seq_lens    [B]                                 int32
 *   o           [B, Hq, d]                          bf16 (out)
 *   lse         [B, Hq]                             float (out)
 *   workspace   >= fa_paged_decode_workspace_size(B, Hq, d, page_size, max_seq_len) bytes
 *
 * Token t (0 <= t < seq_lens[b]) of sequence b is stored in page
 * block_table[b][t / page_size], slot t % page_size, of both pools. The
 * query sees every cached token (no mask). Slots at or past seq_lens[b] in the
 * sequence's last page, and table entries past its last page, are never used
 * (they may hold anything, e.g. -1 in the table).
 * Caller guarantees: 0 <= seq_lens[b] <= min(max_seq_len,
 * max_pages_per_seq * page_size), and every used table entry is in
 * [0, num_pages). seq_lens[b] == 0 gives O = 0 and LSE = -inf.
 * Sizes: B, Hq, Hkv >= 1, Hq % Hkv == 0, d in {64, 128}, page_size == 16,
 * num_pages >= 1, max_pages_per_seq >= 1, 1 <= max_seq_len <=
 * max_pages_per_seq * page_size. B == 0 is a no-op returning FA_OK.
 * The workspace is scratch owned by the caller; its contents on entry do not
 * matter and are clobbered. Calls that share a workspace must be ordered (one
 * stream).
 * Returns FA_OK once both kernels (split, combine) are enqueued.
 */
int fa_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, int page_size,
                    void* o, float* lse,
                    int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                    int max_seq_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It computes exactly what fa_paged_decode
 * computes, with the same kernels (bit-identical results), and keeps its
 * split-K partials in the library's own scratch: a static device array of
 * FA_PAGED_DECODE_NOALLOC_MAX_BYTES per device, which each device that the
 * library runs on holds until the process ends. It calls no allocating
 * routine.
 *
 * Arguments, caller guarantees and status codes as for fa_paged_decode,
 * except: FA_ERR_WORKSPACE when the partials these sizes need exceed
 * FA_PAGED_DECODE_NOALLOC_MAX_BYTES (B * Hq * S * (d + 1) * 4 bytes, S the
 * number of 2048- or 4096-token splits of max_seq_len; 64 sequences of
 * 32768 tokens with Hq = 64, Hkv = 8, d = 128 need 16.9 MB), and FA_ERR_HIP
 * when the scratch cannot be located. The first call on each device looks the
 * array up (hipGetSymbolAddress, with that device current): make it outside
 * graph capture. The call runs on the current device; `stream` must belong to
 * it.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents (nothing in it needs to start at zero: each call writes
 * every partial it reads). Calls that overlap on one device -- on different
 * streams, or from several threads without ordering -- race on it and give
 * undefined results; order them on one stream.
 */
#define FA_PAGED_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int fa_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens, int page_size,
                            void* o, float* lse,
                            int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                            int max_seq_len, float scale, void* stream);

/*
 * Paged (chunked) prefill: for every sequence, a chunk of new queries against
 * its paged KV cache -- the attention equation computed with the page layout
 * of the decode path. Source: "FlashAttention" glossary (polydesk.ai),
 * section "FlashAttention vs PagedAttention" (the two are complementary: one
 * computes attention, the other stores the KV cache, used together); page
 * layout and lookup table as for fa_paged_decode.
 *
 *   q            [total_q, Hq, d]                    bf16 (packed rows)
 *   k_pool       [num_pages, Hkv, page_size, d]      bf16
 *   v_pool       [num_pages, Hkv, page_size, d]      bf16
 *   block_table  [B, max_pages_per_seq]              int32
 *   seq_lens     [B]                                 int32 (keys of each sequence)
 *   cu_seqlens_q [B + 1]                             int32 (row offsets into q)
 *   o            [total_q, Hq, d]                    bf16 (out)
 *   lse          [total_q, Hq]                       float (out)
 *
 * Sequence b owns the n_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] query rows
 * starting at row cu_seqlens_q[b], and the L_b = seq_lens[b] keys / values
 * stored as for fa_paged_decode (token t in page block_table[b][t/page_size],
 * slot t % page_size). The queries are the last n_b tokens of the sequence:
 * causal != 0 lets query i (0 <= i < n_b) see key j iff j <= i + (L_b - n_b)
 * (the causal diagonal aligned to the last query and key, as in fa_forward);
 * causal == 0 lets every query see all L_b keys. So the new tokens' own K/V
 * must already be in the pools.
 * Caller guarantees (device data, not checked): cu_seqlens_q non-decreasing
 * with every n_b <= max_q_len; 0 <= L_b <= max_pages_per_seq * page_size;
 * every used table entry in [0, num_pages). Rows with no visible key get
 * O = 0 and LSE = -inf (e.g. n_b > L_b, or L_b == 0).
 * Sizes: B >= 0 (0 is a no-op), Hq, Hkv >= 1, Hq % Hkv == 0, d in {64, 128},
 * page_size == 16, num_pages >= 1, max_pages_per_seq >= 1, max_q_len >= 0
 * (0 is a no-op). No workspace: the kernel allocates nothing.
 * Returns FA_OK once the kernel is enqueued, or a negative fa_status.
 */
int fa_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                     int page_size, void* o, float* lse,
                     int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                     int max_q_len, int causal, float scale, void* stream);

/*
 * Paged (chunked) prefill with a sliding window: fa_paged_prefill with the
 * two bounds of fa_forward_window. Sources: as for fa_paged_prefill, and for
 * the window "FlashAttention" glossary (polydesk.ai), section "FlashAttention
 * et attention block-sparse", and "FlashAttention et PagedAttention : à quoi
 * servent-elles ?" (ranksignal.fr), section "Trois idées reçues à écarter"
 * (a sliding window looks only at the most recent tokens; here over the
 * paged cache).
 *
 * Same tensors, sizes, guarantees and errors as fa_paged_prefill. Query i of
 * sequence b sits at key position p = i + (L_b - n_b) and sees key j iff
 *     (window_left  < 0 or j >= p - window_left) and
 *     (window_right < 0 or j <= p + window_right) and
 *     (causal == 0 or j <= p) and j < L_b.
 * -1 means unbounded; causal != 0 forces the right bound to 0. Pages wholly
 * outside every row's window of a workgroup are never read (nor their table
 * entries). Rows with no visible key get O = 0 and LSE = -inf.
 * Returns FA_ERR_WINDOW for a bound below -1; otherwise as fa_paged_prefill.
 */
int fa_paged_prefill_window(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                            int page_size, void* o, float* lse,
                            int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                            int max_q_len, int causal, int window_left, int window_right, float scale,
                            void* stream);

/* Static, human-readable text for an fa_status value. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
