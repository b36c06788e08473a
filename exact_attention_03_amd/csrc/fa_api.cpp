// C-ABI entry points of libfa: argument validation on the host (before any
// HIP call), then one enqueue on the caller's stream. See include/fa.h for
// the contract of each function.
#include "../../include/fa.h"

#include <cmath>
#include <cstdint>

#include "fa_kernels.h"

namespace {

static_assert(FA_SPARSE_BLOCK == fa::kSparseMaskBlock && FA_SPARSE_MAX_KEY_BLOCKS == fa::kSparseMaxKeyBlocks,
              "public and kernel block-sparse limits agree");
static_assert(FA_PAGED_DECODE_NOALLOC_MAX_BYTES == fa::kNoAllocScratchBytes,
              "public and library limits of the allocation-free decode agree");

constexpr long long kMaxElems = 1LL << 40;
constexpr int kMaxSeq = 1 << 30;

bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

int validate_forward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || Nq >= kMaxSeq || Nk >= kMaxSeq) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if (!scale_ok(scale)) return FA_ERR_SCALE;
    if ((long long)B * Hq * Nq * d >= kMaxElems || (long long)B * Hkv * Nk * d >= kMaxElems) return FA_ERR_SHAPE;
    if (Nq > 0 && (q == nullptr || o == nullptr || lse == nullptr)) return FA_ERR_NULL;
    if (Nk > 0 && Nq > 0 && (k == nullptr || v == nullptr)) return FA_ERR_NULL;
    return FA_OK;
}

// Two floats per query row: rowsum(dO * O), then the LSE in exp2 units.
size_t backward_workspace_bytes(long long B, long long Hq, long long Nq) { return (size_t)(B * Hq * Nq) * 8; }

// Steps of the block-sparse dK/dV walk of one key block: query heads per K/V
// head times 64-query tiles.
long long sparse_backward_steps(int Hq, int Hkv, int Nq) { return (long long)(Hq / Hkv) * ((Nq + 63) / 64); }

size_t decode_workspace_bytes(long long B, long long Hq, long long d, int max_seq_len) {
    const long long S = fa::decode_num_splits(max_seq_len);
    return (size_t)(B * Hq * S * (d + 1) * 4);
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               int causal, float scale, void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    if (Nq == 0) return FA_OK;
    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale, -1, causal ? 0 : -1};
    return fa::launch_forward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_window(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      int causal, int window_left, int window_right, float scale, void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_WINDOW;
    if (Nq == 0) return FA_OK;
    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale, window_left,
                  causal ? 0 : window_right};
    return fa::launch_forward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                            const uint8_t* block_mask, long long mask_stride_b, long long mask_stride_h,
                            float scale, void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    const long long n_kb = ((long long)Nk + fa::kSparseMaskBlock - 1) / fa::kSparseMaskBlock;
    if (n_kb > fa::kSparseMaxKeyBlocks || mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_SHAPE;
    if (Nq == 0) return FA_OK;
    if (block_mask == nullptr) return FA_ERR_NULL;
    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale, -1, causal ? 0 : -1,
                  block_mask, mask_stride_b, mask_stride_h};
    return fa::launch_forward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_quantize_fp8(const void* x, uint8_t* codes, float* scales, int B, int H, int N, int d, int block_rows,
                    void* stream) {
    if (B < 1 || H < 1 || N < 0 || N >= kMaxSeq || block_rows < 1) return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if ((long long)B * H * N * d >= kMaxElems) return FA_ERR_SHAPE;
    if (N == 0) return FA_OK;
    if (!x || !codes || !scales) return FA_ERR_NULL;
    return fa::launch_quantize_fp8(x, codes, scales, B, H, N, d, block_rows, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? FA_OK
               : FA_ERR_HIP;
}

int fa_quantize_fp8_incoherent(const void* x, const int8_t* signs, uint8_t* codes, float* scales, int B, int H,
                               int N, int d, int block_rows, void* stream) {
    if (B < 1 || H < 1 || N < 0 || N >= kMaxSeq || block_rows < 1) return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if ((long long)B * H * N * d >= kMaxElems) return FA_ERR_SHAPE;
    if (N == 0) return FA_OK;
    if (!x || !signs || !codes || !scales) return FA_ERR_NULL;
    return fa::launch_quantize_fp8_incoherent(x, signs, codes, scales, B, H, N, d, block_rows,
                                              static_cast<hipStream_t>(stream)) == hipSuccess
               ? FA_OK
               : FA_ERR_HIP;
}

int fa_forward_fp8(const uint8_t* q, const float* q_scales, const uint8_t* k, const float* k_scales,
                   const uint8_t* v, const float* v_scales, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, int causal, float scale, void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    if (Nq == 0) return FA_OK;
    if (!q_scales || (Nk > 0 && (!k_scales || !v_scales))) return FA_ERR_NULL;
    fa::Fp8Args a{q, k, v, q_scales, k_scales, v_scales, o, lse, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale};
    return fa::launch_forward_fp8(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_backward_workspace_size(int B, int Hq, int Nq) {
    if (B < 0 || Hq < 1 || Nq < 0 || Nq >= kMaxSeq) return 0;
    return backward_workspace_bytes(B, Hq, Nq);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                void* workspace, size_t workspace_bytes, void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    if (Nq > 0 && (dout == nullptr || dq == nullptr)) return FA_ERR_NULL;
    if (Nk > 0 && (dk == nullptr || dv == nullptr || k == nullptr || v == nullptr)) return FA_ERR_NULL;
    if (Nq == 0 && Nk == 0) return FA_OK;
    if (Nq > 0 && (workspace == nullptr || workspace_bytes < backward_workspace_bytes(B, Hq, Nq))) return FA_ERR_WORKSPACE;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale, workspace};
    return fa::launch_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       int causal, int window_left, int window_right, float scale, void* workspace,
                       size_t workspace_bytes, void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_WINDOW;
    if (Nq > 0 && (dout == nullptr || dq == nullptr)) return FA_ERR_NULL;
    if (Nk > 0 && (dk == nullptr || dv == nullptr || k == nullptr || v == nullptr)) return FA_ERR_NULL;
    if (Nq == 0 && Nk == 0) return FA_OK;
    if (Nq > 0 && (workspace == nullptr || workspace_bytes < backward_workspace_bytes(B, Hq, Nq))) return FA_ERR_WORKSPACE;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale, workspace,
                  window_left, window_right};
    return fa::launch_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_backward_block_sparse_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Nq < 0 || Nk < 0 || Nq >= kMaxSeq || Nk >= kMaxSeq ||
        !head_dim_ok(d))
        return 0;
    if (B == 0 || sparse_backward_steps(Hq, Hkv, Nq) > fa::kSparseMaxBackwardSteps) return 0;
    return fa::sparse_backward_plan(B, Hq, Hkv, Nq, Nk, d).bytes;
}

int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk,
                             int d, int causal, const uint8_t* block_mask, long long mask_stride_b,
                             long long mask_stride_h, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
    const int st = validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale);
    if (st != FA_OK) return st;
    const long long n_kb = ((long long)Nk + fa::kSparseMaskBlock - 1) / fa::kSparseMaskBlock;
    if (n_kb > fa::kSparseMaxKeyBlocks || mask_stride_b < 0 || mask_stride_h < 0) return FA_ERR_SHAPE;
    if (sparse_backward_steps(Hq, Hkv, Nq) > fa::kSparseMaxBackwardSteps) return FA_ERR_SHAPE;
    if (Nq > 0 && (dout == nullptr || dq == nullptr || block_mask == nullptr)) return FA_ERR_NULL;
    if (Nk > 0 && (dk == nullptr || dv == nullptr || k == nullptr || v == nullptr)) return FA_ERR_NULL;
    if (Nq == 0 && Nk == 0) return FA_OK;
    const size_t need = fa::sparse_backward_plan(B, Hq, Hkv, Nq, Nk, d).bytes;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal ? 1 : 0, scale, workspace,
                  -1, -1, block_mask, mask_stride_b, mask_stride_h};
    return fa::launch_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_paged_decode_workspace_size(int B, int Hq, int d, int page_size, int max_seq_len) {
    if (B < 0 || Hq < 1 || !head_dim_ok(d) || page_size != 16 || max_seq_len < 1) return 0;
    return decode_workspace_bytes(B, Hq, d, max_seq_len);
}

}  // extern "C"

namespace {

// Arguments of the paged decode without its workspace; FA_OK also for B == 0
// (nothing to do).
int validate_paged_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, int page_size, const void* o, const float* lse, int B, int Hq,
                          int Hkv, int d, int num_pages, int max_pages_per_seq, int max_seq_len, float scale) {
    if (B < 0 || Hq < 1 || Hkv < 1 || num_pages < 1 || max_pages_per_seq < 1 || max_seq_len < 1)
        return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if (page_size != 16) return FA_ERR_PAGESIZE;
    if ((long long)max_pages_per_seq * page_size < max_seq_len || max_seq_len >= kMaxSeq) return FA_ERR_SHAPE;
    if ((long long)num_pages * Hkv * page_size * d >= kMaxElems || (long long)B * Hq * d >= kMaxElems ||
        (long long)B * max_pages_per_seq >= kMaxElems)
        return FA_ERR_SHAPE;
    if (B > 65535 || (long long)Hkv * ((Hq / Hkv + 15) / 16) > 65535) return FA_ERR_SHAPE;  // grid y/z limits
    if (!scale_ok(scale)) return FA_ERR_SCALE;
    if (B == 0) return FA_OK;
    if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o || !lse) return FA_ERR_NULL;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const int32_t* seq_lens, int page_size,
                    void* o, float* lse,
                    int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                    int max_seq_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
    const int st = validate_paged_decode(q, k_pool, v_pool, block_table, seq_lens, page_size, o, lse, B, Hq, Hkv, d,
                                         num_pages, max_pages_per_seq, max_seq_len, scale);
    if (st != FA_OK || B == 0) return st;
    if (workspace == nullptr || workspace_bytes < decode_workspace_bytes(B, Hq, d, max_seq_len))
        return FA_ERR_WORKSPACE;
    fa::DecodeArgs a{q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, d, page_size,
                     num_pages, max_pages_per_seq, max_seq_len, scale, workspace};
    return fa::launch_paged_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens, int page_size,
                            void* o, float* lse,
                            int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                            int max_seq_len, float scale, void* stream) {
    const int st = validate_paged_decode(q, k_pool, v_pool, block_table, seq_lens, page_size, o, lse, B, Hq, Hkv, d,
                                         num_pages, max_pages_per_seq, max_seq_len, scale);
    if (st != FA_OK || B == 0) return st;
    if (fa::paged_decode_partials_bytes(B, Hq, Hkv, d, max_seq_len) > fa::kNoAllocScratchBytes)
        return FA_ERR_WORKSPACE;
    void* scratch = nullptr;
    if (fa::noalloc_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
    fa::DecodeArgs a{q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, d, page_size,
                     num_pages, max_pages_per_seq, max_seq_len, scale, scratch};
    return fa::launch_paged_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

// Arguments of the paged chunked prefill (with or without a window); FA_OK
// also when there is nothing to do (then *empty is set).
int validate_paged_prefill(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* cu_seqlens_q, int page_size, const void* o,
                           const float* lse, int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                           int max_q_len, float scale, bool* empty) {
    *empty = false;
    if (B < 0 || Hq < 1 || Hkv < 1 || num_pages < 1 || max_pages_per_seq < 1 || max_q_len < 0 ||
        max_q_len >= kMaxSeq)
        return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if (page_size != 16) return FA_ERR_PAGESIZE;
    if ((long long)num_pages * Hkv * page_size * d >= kMaxElems || (long long)B * max_pages_per_seq >= kMaxElems ||
        (long long)max_pages_per_seq * page_size >= kMaxSeq || (long long)B * max_q_len * Hq * d >= kMaxElems)
        return FA_ERR_SHAPE;
    if ((long long)B * Hq * ((max_q_len + 31) / 32) > 0x7fffffffLL) return FA_ERR_SHAPE;  // grid size
    if (!scale_ok(scale)) return FA_ERR_SCALE;
    if (B == 0 || max_q_len == 0) {
        *empty = true;
        return FA_OK;
    }
    if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !cu_seqlens_q || !o || !lse) return FA_ERR_NULL;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_paged_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                     int page_size, void* o, float* lse,
                     int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                     int max_q_len, int causal, float scale, void* stream) {
    bool empty = false;
    const int st = validate_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, page_size, o, lse,
                                          B, Hq, Hkv, d, num_pages, max_pages_per_seq, max_q_len, scale, &empty);
    if (st != FA_OK || empty) return st;
    fa::PagedPrefillArgs a{q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse,
                           B, Hq, Hkv, d, num_pages, max_pages_per_seq, max_q_len, causal ? 1 : 0, scale};
    return fa::launch_paged_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_paged_prefill_window(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                            int page_size, void* o, float* lse,
                            int B, int Hq, int Hkv, int d, int num_pages, int max_pages_per_seq,
                            int max_q_len, int causal, int window_left, int window_right, float scale,
                            void* stream) {
    bool empty = false;
    const int st = validate_paged_prefill(q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, page_size, o, lse,
                                          B, Hq, Hkv, d, num_pages, max_pages_per_seq, max_q_len, scale, &empty);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_WINDOW;
    if (empty) return FA_OK;
    fa::PagedPrefillArgs a{q, k_pool, v_pool, block_table, seq_lens, cu_seqlens_q, o, lse,
                           B, Hq, Hkv, d, num_pages, max_pages_per_seq, max_q_len, causal ? 1 : 0, scale,
                           window_left, window_right};
    return fa::launch_paged_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "a size is out of range";
        case FA_ERR_GQA: return "Hq is not a positive multiple of Hkv";
        case FA_ERR_HEADDIM: return "head dimension not supported (64 and 128 are)";
        case FA_ERR_PAGESIZE: return "page size not supported (16 is)";
        case FA_ERR_WORKSPACE: return "workspace missing or too small";
        case FA_ERR_SCALE: return "scale must be finite and positive";
        case FA_ERR_WINDOW: return "window bounds must be -1 (none) or >= 0";
        case FA_ERR_HIP: return "HIP runtime error while enqueuing";
        default: return "unknown status";
    }
}

}  // extern "C"
