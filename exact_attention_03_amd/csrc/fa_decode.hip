// Paged GQA decode for gfx950: one query token per sequence against a KV cache
// stored in fixed-size pages found through a block table, with split-K over
// the cached tokens and a log-sum-exp combine of the partial results.
//
// Sources (pages cited by title and section): the paged cache layout and its
// lookup table, with the computation unchanged -- "FlashAttention et
// PagedAttention : a quoi servent-elles ?", section "PagedAttention : ranger
// par pages plutot que d'un seul tenant"; the running max / sum statistics
// that make partial softmax results mergeable -- "FlashAttention" glossary
// (polydesk.ai), section "L'idee cle : IO-awareness"; GQA head sharing --
// "Variantes d'attention", "Termes employes sur cette page".
//
// gfx950 mapping (this file's own design):
//   * Split kernel: one workgroup (4 waves) per (split, K/V head, sequence).
//     A split is 2048 tokens (128 pages), or 4096 at d = 128 when that grid
//     still has >= 2048 workgroups (measured ~2% faster on a 64-sequence
//     batch: fewer partials to write and merge). The grid is split-major with the K/V head
//     fastest: workgroups running together read all K/V heads of the same
//     pages, i.e. neighbouring 4 KiB blocks of each page, which keeps HBM
//     accesses local (this ordering alone is worth ~17% of bandwidth here).
//     Splits past the sequence end exit at once. The split's block-table
//     entries are fetched with one load per lane and register and broadcast
//     with readlane, so page addresses never wait on a dependent scalar load
//     inside the loop.
//   * Each wave takes pages w, w+4, w+8, ...; K and V of the next page are
//     loaded into a second, statically named register set while the current
//     page is computed (the prefetch is unconditional so that the compiler's
//     wait counts stay exact). Scores S^T = K q^T use
//     v_mfma_f32_16x16x32_bf16 with K straight from registers as the A
//     operand (16 tokens x 8 dims per lane) and the G query heads of the K/V
//     head as the 16 columns; every lane then holds 4 tokens of one head,
//     which is exactly the B operand of O^T += V^T P^T with
//     v_mfma_f32_16x16x16_bf16 (16 tokens deep). V goes through the wave's
//     own LDS page buffer and comes back transposed (ds_read_b64_tr_b16).
//   * Slots past the sequence end get weight 0 and are staged as 0.
//   * The four waves' (max, sum, O) states are merged through LDS; the split
//     writes a normalised fp32 partial and its LSE, or the final bf16 output
//     directly when the sequence fits in one split.
//   * Combine kernel: one wave per (sequence, query head) merges the splits
//     in a fixed order (deterministic): LSE = M + ln sum exp(LSE_s - M),
//     O = sum exp(LSE_s - LSE) O_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa_kernels.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;

struct DecParams {
    const uint16_t* q;
    const uint16_t* kp;
    const uint16_t* vp;
    const int32_t* bt;
    const int32_t* seq_lens;
    uint16_t* o;
    float* lse;
    float* part_o;    // [B, Hq, S, D]
    float* part_lse;  // [B, Hq, S]
    int B, Hq, Hkv, G, n_hgrp, S, maxp;
    int split;  // tokens per split (SPLIT of the split kernel)
    float scale_log2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float xor_lanes(float x, int m) { return __shfl_xor(x, m, 64); }

// XOR swizzle of the 16-byte chunks of a staged V row (token): the
// transposing reads of 4 consecutive tokens x 4 consecutive chunks hit
// distinct bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// K and V of one page (16 tokens) of one K/V head, in registers: K in the
// MFMA A-operand layout (token = lane % 16, 8 dims), V as the page's 16-byte
// chunks i*64 + lane (token (i*64 + lane) / (D/8)).
template <int D>
struct PageRegs {
    u32x4 k[D / 32];
    u32x4 v[D / 32];
};

template <int D, int NB>
__device__ __forceinline__ void load_page(PageRegs<D>& pr, const DecParams& p, const int (&bt_entry)[NB],
                                          int lp, int g, int lane) {
    constexpr int KS = D / 32;
    int e = bt_entry[0];
#pragma unroll
    for (int r = 1; r < NB; ++r) e = (lp >> 6) == r ? bt_entry[r] : e;
    const int pg = __builtin_amdgcn_readlane(e, lp & 63);
    const size_t head_stride = (size_t)kPage * D;
    const size_t off = (size_t)pg * p.Hkv * head_stride + (size_t)g * head_stride;
    const uint16_t* kb = p.kp + off;
    const uint16_t* vb = p.vp + off;
    const int lrow = lane & 15, lgrp = lane >> 4;
    // Every K/V byte is read once per call, and a serving batch's KV cache
    // is far larger than L2 and the MALL: non-temporal loads stream it past
    // them instead of evicting lines that are reused (measured +1.6-1.9%
    // bandwidth, identical results).
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        pr.k[ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + lrow * D + ks * 32 + lgrp * 8));
#pragma unroll
    for (int i = 0; i < KS; ++i)
        pr.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (size_t)(i * 64 + lane) * 8));
}

template <int D, int SPLIT>
__global__ __launch_bounds__(kThreads) void fa_decode_split_kernel(DecParams p) {
    constexpr int kBtRegs = SPLIT / kPage / 64;  // block-table entries per lane
    constexpr int KS = D / 32;   // 32-dim k-steps of K q^T
    constexpr int DB = D / 16;   // 16-dim blocks of O^T
    constexpr int CH = D / 8;    // 16-byte chunks per token row
    constexpr int kPageBytes = kPage * D * 2;
    constexpr int kMergeBytes = 4 * (D * 16 + 32) * 4;
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * kPageBytes > kMergeBytes ? 4 * kPageBytes : kMergeBytes];

    const int split = blockIdx.z;
    const int g = blockIdx.x % p.Hkv;
    const int hgrp = blockIdx.y;
    const int b = blockIdx.x / p.Hkv;
    const int L = p.seq_lens[b];
    const int tok0 = split * SPLIT;
    if (tok0 >= L) return;
    const int tok1 = min(L, tok0 + SPLIT);
    const int pg_begin = tok0 / kPage;
    const int n_pages = (tok1 - tok0 + kPage - 1) / kPage;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int hcol = hgrp * 16 + lrow;  // query head (within the group) of this lane's column
    const bool hvalid = hcol < p.G;

    // Block-table entries of this split: lane i of register r holds page
    // 64*r + i of the split.
    int bt_entry[kBtRegs];
#pragma unroll
    for (int r = 0; r < kBtRegs; ++r) {
        const int lp = 64 * r + lane;
        bt_entry[r] = (lp < n_pages) ? p.bt[(size_t)b * p.maxp + pg_begin + lp] : 0;
    }

    // q^T fragments (B operand): column = head, 8 dims per lane.
    bf16x8 qf[KS];
    {
        const uint16_t* qp = p.q + ((size_t)b * p.Hq + (size_t)g * p.G + (hvalid ? hcol : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (hvalid) x = *reinterpret_cast<const u32x4*>(qp + ks * 32 + lgrp * 8);
            qf[ks] = as_bf16x8(x);
        }
    }

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref = -INFINITY, lsum = 0.0f;

    char* vst = smem_raw + wave * kPageBytes;  // this wave's V staging: one page, token rows
    int wr_off[KS];  // staging offset of this lane's V chunk per load slot
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        const int row = (i * 64 + lane) / CH, c = (i * 64 + lane) % CH;
        wr_off[i] = row * (D * 2) + ((c ^ vswz<D>(row)) << 4);
    }
    int rd_off[DB];  // this lane's transposing-read address per 16-dim block
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int j = lane & 15;
        const int row = 4 * lgrp + (j >> 2);
        const int dim = db * 16 + 4 * (j & 3);
        rd_off[db] = row * (D * 2) + (((dim >> 3) ^ vswz<D>(row)) << 4) + (dim & 7) * 2;
    }

    auto compute = [&](const PageRegs<D>& pr, int lp) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pr.k[ks]), qf[ks], sc, 0, 0, 0);
        // Stage V; slots past the sequence end may hold any bits (even NaN):
        // they get weight 0 below and are staged as 0 so 0 * NaN cannot occur.
        const int valid = tok1 - (tok0 + lp * kPage);
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < KS; ++i)
            *reinterpret_cast<u32x4*>(vst + wr_off[i]) = ((i * 64 + lane) / CH) < valid ? pr.v[i] : z;
        // Mask tokens past the sequence end.
        const int t = tok0 + lp * kPage + lgrp * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (t + r >= tok1) sc[r] = -INFINITY;
        float m = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        m = fmaxf(m, xor_lanes(m, 16));
        m = fmaxf(m, xor_lanes(m, 32));
        const float mx = m * p.scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > mref + kRescaleSlack) != 0) {
            const float mnew = fmaxf(mref, mx);
            const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mref - mnew);
            mref = mnew;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        const float ref = (mref == -INFINITY) ? 0.0f : mref;
        bf16x4 pf;
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], p.scale_log2, -ref));
            acc += x;
            pf[r] = (__bf16)x;
        }
        lsum += acc;
        // O^T += V^T P^T (16x16x16): A row = dim 16*db + lrow, k = tokens
        // 4*lgrp..+3, one transposing read of the staged page (the wave's own
        // LDS region; its writes above are visible to its reads).
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vst + rd_off[db]));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vt),
                                                                __builtin_bit_cast(s16x4, pf), oacc[db], 0, 0, 0);
        }
    };

    // Pages w, w+4, w+8, ... alternate between two statically named register
    // sets, so the next page's loads are in flight while this one computes.
    // The prefetch is unconditional (past the wave's last page it re-reads
    // that page): a conditional load would make the compiler wait for the
    // current page as if nothing newer were in flight.
    // Pages are processed in pairs with both computations unconditional (an
    // exit between them would make the compiler duplicate the accumulators);
    // an odd last page is computed after the loop from ra, which the last
    // pair prefetched.
    const int nw = wave < n_pages ? (n_pages - wave + 3) / 4 : 0;  // pages of this wave
    const int last_lp = wave + 4 * (nw - 1);
    PageRegs<D> ra, rb;
    if (nw > 0) {
        load_page<D, kBtRegs>(ra, p, bt_entry, wave, g, lane);
        int i = 0;
        for (; i + 2 <= nw; i += 2) {
            const int lp = wave + 4 * i;
            load_page<D, kBtRegs>(rb, p, bt_entry, lp + 4, g, lane);
            compute(ra, lp);
            load_page<D, kBtRegs>(ra, p, bt_entry, min(lp + 8, last_lp), g, lane);
            compute(rb, lp + 4);
        }
        if (i < nw) compute(ra, wave + 4 * i);
    }

    // ---- merge the 4 waves: (mref, l, O^T) per head column ----
    lsum += xor_lanes(lsum, 16);
    lsum += xor_lanes(lsum, 32);
    __syncthreads();  // V staging is free from here on
    float* st_o = reinterpret_cast<float*>(smem_raw);      // [4 waves][D][16]
    float* st_m = st_o + 4 * D * 16;                       // [4 waves][16]
    float* st_l = st_m + 4 * 16;                           // [4 waves][16]
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) st_o[(wave * D + db * 16 + lgrp * 4 + r) * 16 + lrow] = oacc[db][r];
    if (lgrp == 0) {
        st_m[wave * 16 + lrow] = mref;
        st_l[wave * 16 + lrow] = lsum;
    }
    __syncthreads();

    const int n_splits = (L + SPLIT - 1) / SPLIT;
    const int ncols = min(16, p.G - hgrp * 16);
    for (int idx = tid; idx < ncols * D; idx += kThreads) {
        const int c = idx / D, dim = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, st_m[w * 16 + c]);
        const float Mz = (M == -INFINITY) ? 0.0f : M;
        float l = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sc = (st_m[w * 16 + c] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st_m[w * 16 + c] - Mz);
            l += st_l[w * 16 + c] * sc;
            o += st_o[(w * D + dim) * 16 + c] * sc;
        }
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        const int h = g * p.G + hgrp * 16 + c;
        const size_t bh = (size_t)b * p.Hq + h;
        const float lse = l > 0.0f ? M * kLn2 + logf(l) : -INFINITY;
        if (n_splits == 1) {
            p.o[bh * D + dim] = __builtin_bit_cast(uint16_t, (__bf16)(o * inv));
            if (dim == 0) p.lse[bh] = lse;
        } else {
            p.part_o[(bh * p.S + split) * D + dim] = o * inv;
            if (dim == 0) p.part_lse[bh * p.S + split] = lse;
        }
    }
}

// Wave-wide reductions (all 64 lanes get the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// One wave per (sequence, query head). Lane s holds LSE_s of split s (up to
// 64 splits per pass); the weights exp(LSE_s - LSE) are broadcast with
// readlane and the partial rows are summed in split order (deterministic).
template <int D>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(DecParams p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long bh = (long long)blockIdx.x * 4 + wave;
    if (bh >= (long long)p.B * p.Hq) return;
    const int b = (int)(bh / p.Hq);
    const int L = p.seq_lens[b];
    const int n = (L + p.split - 1) / p.split;
    constexpr int DPL = D / 64;  // dims per lane
    if (n == 1) return;          // written by the split kernel
    if (n == 0) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) p.o[bh * D + lane * DPL + e] = 0;
        if (lane == 0) p.lse[bh] = -INFINITY;
        return;
    }
    const float* pl = p.part_lse + bh * p.S;
    // Pass 1: M = max_s LSE_s and den = sum_s exp(LSE_s - M).
    float M = -INFINITY;
    for (int s0 = 0; s0 < n; s0 += 64) M = fmaxf(M, wave_max(s0 + lane < n ? pl[s0 + lane] : -INFINITY));
    const float Mz = (M == -INFINITY) ? 0.0f : M;
    float den = 0.0f;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const float x = s0 + lane < n ? pl[s0 + lane] : -INFINITY;
        den += wave_sum(x == -INFINITY ? 0.0f : __expf(x - Mz));
    }
    const float lse = den > 0.0f ? Mz + logf(den) : -INFINITY;
    // Pass 2: O = sum_s exp(LSE_s - LSE) O_s, weights broadcast from lane s.
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
    const float* po = p.part_o + (size_t)bh * p.S * D + lane * DPL;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const float x = s0 + lane < n ? pl[s0 + lane] : -INFINITY;
        const float wl = (x == -INFINITY || den == 0.0f) ? 0.0f : __expf(x - lse);
        const int cnt = min(64, n - s0);
        int s = 0;
        for (; s + 4 <= cnt; s += 4) {  // four partial rows in flight
            float v[4][DPL];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < DPL; ++e) v[u][e] = po[(size_t)(s0 + s + u) * D + e];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s + u));
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[e] += w * v[u][e];
            }
        }
        for (; s < cnt; ++s) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] += w * po[(size_t)(s0 + s) * D + e];
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) p.o[bh * D + lane * DPL + e] = __builtin_bit_cast(uint16_t, (__bf16)acc[e]);
    if (lane == 0) p.lse[bh] = lse;
}

template <int D, int SPLIT>
hipError_t launch_t(const DecParams& p, hipStream_t stream) {
    dim3 grid(p.B * p.Hkv, p.n_hgrp, p.S);
    const long long nbh = (long long)p.B * p.Hq;
    if (trace_on()) {
        trace("fa_decode_split_kernel<d=%d, split=%d> grid=(%d,%d,%d) block=%d", D, SPLIT, p.B * p.Hkv, p.n_hgrp,
              p.S, kThreads);
        trace("fa_decode_combine_kernel<d=%d> grid=%lld block=256", D, (nbh + 3) / 4);
    }
    hipLaunchKernelGGL((fa_decode_split_kernel<D, SPLIT>), grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fa_decode_combine_kernel<D>), dim3((unsigned)((nbh + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// Split length for a call: d = 128 takes the long split when its grid still
// gives every CU several workgroups (d = 64 would keep its table entries in
// scratch); the workspace (sized for the short split) holds either layout.
struct SplitPlan {
    bool long_split;
    int split, S;
};
SplitPlan plan_splits(int B, int Hq, int Hkv, int d, int max_seq_len) {
    const int n_hgrp = (Hq / Hkv + 15) / 16;
    const int s_long = (max_seq_len + kDecodeLongSplitTokens - 1) / kDecodeLongSplitTokens;
    const bool long_split = d == 128 && (long long)B * Hkv * n_hgrp * s_long >= kDecodeLongSplitMinGroups;
    return {long_split, long_split ? kDecodeLongSplitTokens : kDecodeSplitTokens,
            long_split ? s_long : decode_num_splits(max_seq_len)};
}

// The allocation-free entry point's scratch (split-K partials): one array per
// device, which every call on that device shares and which keeps the last
// call's contents. Host code never uses this name as an address; it uses the
// device address from hipGetSymbolAddress (noalloc_scratch).
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

size_t paged_decode_partials_bytes(int B, int Hq, int Hkv, int d, int max_seq_len) {
    const SplitPlan sp = plan_splits(B, Hq, Hkv, d, max_seq_len);
    return (size_t)B * Hq * sp.S * (d + 1) * sizeof(float);
}

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
    DecParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.kp = static_cast<const uint16_t*>(a.k_pool);
    p.vp = static_cast<const uint16_t*>(a.v_pool);
    p.bt = a.block_table;
    p.seq_lens = a.seq_lens;
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.n_hgrp = (p.G + 15) / 16;
    const SplitPlan sp = plan_splits(a.B, a.Hq, a.Hkv, a.d, a.max_seq_len);
    const bool long_split = sp.long_split;
    p.split = sp.split;
    p.S = sp.S;
    p.maxp = a.max_pages_per_seq;
    p.scale_log2 = a.scale * kLog2e;
    p.part_o = static_cast<float*>(a.workspace);
    p.part_lse = p.part_o + (size_t)a.B * a.Hq * p.S * a.d;
    if (a.B == 0) return hipSuccess;
    if (long_split) return launch_t<128, kDecodeLongSplitTokens>(p, stream);
    return a.d == 128 ? launch_t<128, kDecodeSplitTokens>(p, stream) : launch_t<64, kDecodeSplitTokens>(p, stream);
}

}  // namespace fa
