// Internal launch interface between the C-ABI wrapper (fa_api.cpp) and the
// gfx950 kernels. Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk, d;
    int causal;
    float scale;
    int window_left;   // -1: none
    int window_right;  // -1: none (causal uses 0)
    // Block-sparse mask (nullptr: dense): [B, Hq, ceil(Nq/128), ceil(Nk/128)]
    // bytes, batch / head strides in bytes (0 broadcasts).
    const uint8_t* block_mask;
    long long mask_stride_b, mask_stride_h;
};

// Block-sparse mask granularity (queries and keys per block) and the most
// key blocks a mask row may have.
constexpr int kSparseMaskBlock = 128;
constexpr int kSparseMaxKeyBlocks = 4096;
// The block-sparse backward's most steps per key block: (Hq / Hkv) times the
// 64-query tiles of Nq.
constexpr int kSparseMaxBackwardSteps = 131072;

struct DecodeArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* o;
    float* lse;
    int B, Hq, Hkv, d, page_size, num_pages, max_pages_per_seq, max_seq_len;
    float scale;
    void* workspace;
};

struct PagedPrefillArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* cu_seqlens_q;
    void* o;
    float* lse;
    int B, Hq, Hkv, d, num_pages, max_pages_per_seq, max_q_len;
    int causal;
    float scale;
    int window_left = -1;   // sliding window as for fa_forward_window (-1: none)
    int window_right = -1;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    int B, Hq, Hkv, Nq, Nk, d;
    int causal;
    float scale;
    void* workspace;  // 2 * B * Hq * Nq floats
    int window_left = -1;   // sliding window as for fa_forward_window (-1: none)
    int window_right = -1;
    // Block-sparse mask as in FwdArgs (nullptr: dense; never with a window).
    const uint8_t* block_mask = nullptr;
    long long mask_stride_b = 0, mask_stride_h = 0;
};

struct Fp8Args {
    const void* q;  // E4M3 codes
    const void* k;
    const void* v;
    const float* q_scales;  // [B, Hq, ceil(Nq / 128)]
    const float* k_scales;  // [B, Hkv, ceil(Nk / 128)]
    const float* v_scales;  // [B, Hkv]
    void* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk, d;
    int causal;
    float scale;
};

// Tokens handled by one split-K workgroup of the paged decode (a multiple of
// 1024: 64 pages of 16 tokens per block-table register of a wave). Calls
// whose grid stays large with twice that split use the long split (fewer
// partial results, measured faster); the workspace is sized for the short one.
#ifndef FA_DECODE_SPLIT_TOKENS
#define FA_DECODE_SPLIT_TOKENS 2048
#endif
constexpr int kDecodeSplitTokens = FA_DECODE_SPLIT_TOKENS;
constexpr int kDecodeLongSplitTokens = 2 * kDecodeSplitTokens;
constexpr long long kDecodeLongSplitMinGroups = 2048;  // workgroups of the long-split grid
static_assert(kDecodeSplitTokens % 1024 == 0, "split size must be a multiple of 1024 tokens");

inline int decode_num_splits(int max_seq_len) {
    return (max_seq_len + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
}

// FA_TRACE set to a non-empty value other than "0" makes every launch print
// its kernel instantiation, grid and block to stderr: which kernel the
// library chose for a call. No other effect.
inline bool trace_on() {
    static const bool on = [] {
        const char* e = getenv("FA_TRACE");
        return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
    }();
    return on;
}

__attribute__((format(printf, 1, 2))) inline void trace(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    fputs("[fa] ", stderr);
    vfprintf(stderr, fmt, ap);
    fputc('\n', stderr);
    va_end(ap);
}

// Enqueue the prefill kernel; returns hipSuccess or the launch error.
hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);
// Enqueue the prefill kernel in paged mode (query chunks against paged K/V).
hipError_t launch_paged_prefill(const PagedPrefillArgs& a, hipStream_t stream);
// Enqueue the FP8 forward kernel.
hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream);
// Enqueue the block quantizer (bf16 [B, H, N, d] -> E4M3 codes + scales).
hipError_t launch_quantize_fp8(const void* x, void* codes, float* scales, int B, int H, int N, int d, int block_rows,
                               hipStream_t stream);
// Enqueue incoherent processing (rows times diag(signs) H_d / sqrt(d)) fused
// with the block quantizer.
hipError_t launch_quantize_fp8_incoherent(const void* x, const int8_t* signs, void* codes, float* scales, int B, int H,
                                          int N, int d, int block_rows, hipStream_t stream);
// Enqueue the three backward kernels (row sums, dQ, dK / dV).
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);
// Workspace of the block-sparse backward: the per-row values (as
// fa_backward's, first), then, when the dK/dV walk of a key block may be cut
// into up to nseg > 1 runs, one fp32 partial per (batch, K/V head, key block,
// run), one flag per partial and one run count per key block. bytes: the total.
struct SparseBwdPlan {
    int nseg;
    size_t partial_offset, flags_offset, counts_offset, bytes;
};
SparseBwdPlan sparse_backward_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d);
// Enqueue the split-K decode kernel and its combine kernel.
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

// Bytes of split-K partials launch_paged_decode lays out for these sizes (the
// split length it picks): at most the decode workspace size.
size_t paged_decode_partials_bytes(int B, int Hq, int Hkv, int d, int max_seq_len);

// The library's own decode scratch for the allocation-free entry point: a
// static device array of kNoAllocScratchBytes per device. noalloc_scratch()
// returns its device address on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace fa
