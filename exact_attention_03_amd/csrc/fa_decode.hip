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
//   * Split kernel: one workgroup (4 waves) per (split of 1024 tokens = 64
//     pages, K/V head, sequence). Splits past the sequence end exit at once.
//     The 64 block-table entries of a split are fetched by one load per lane
//     and broadcast with readlane, so page addresses never wait on a
//     dependent scalar load inside the loop.
//   * Each wave takes pairs of pages (32 tokens). Scores S^T = K q^T use
//     v_mfma_f32_16x16x32_bf16 with K read straight from global memory into
//     the A operand (16 tokens x 8 dims per lane) and the G query heads of
//     the K/V head as the 16 columns; every lane then holds 4 tokens of one
//     head. The exponentiated scores of the page pair are exactly the B
//     operand of O^T += V^T P^T (16x16x32, 32 tokens deep); V is staged in
//     the wave's own LDS region and read transposed.
//   * The four waves' (max, sum, O) states are merged through LDS; the split
//     writes a normalised fp32 partial and its LSE, or the final bf16 output
//     directly when the sequence fits in one split.
//   * Combine kernel: one wave per (sequence, query head) merges the splits
//     in a fixed order (deterministic): LSE = M + ln sum exp(LSE_s - M),
//     O = sum exp(LSE_s - LSE) O_s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kPage = 16;
constexpr int kSplitPages = kDecodeSplitTokens / kPage;  // 64 = one table entry per lane
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;
static_assert(kSplitPages == 64, "one block-table entry per lane");

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
    float scale_log2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float xor_lanes(float x, int m) { return __shfl_xor(x, m, 64); }

template <int D>
__global__ __launch_bounds__(kThreads) void fa_decode_split_kernel(DecParams p) {
    constexpr int KS = D / 32;   // 32-dim k-steps of K q^T
    constexpr int DB = D / 16;   // 16-dim blocks of O^T
    constexpr int kWaveLds = 2 * kPage * D * 2;  // V bytes of one page pair
    __shared__ __attribute__((aligned(16))) char smem[4 * kWaveLds > 4 * (D * 16 + 32) * 4 ? 4 * kWaveLds : 4 * (D * 16 + 32) * 4];

    const int split = blockIdx.x;
    const int g = blockIdx.y % p.Hkv;
    const int hgrp = blockIdx.y / p.Hkv;
    const int b = blockIdx.z;
    const int L = p.seq_lens[b];
    const int tok0 = split * kDecodeSplitTokens;
    if (tok0 >= L) return;
    const int tok1 = min(L, tok0 + kDecodeSplitTokens);
    const int pg_begin = tok0 / kPage;
    const int n_pages = (tok1 - tok0 + kPage - 1) / kPage;
    const int n_pairs = (n_pages + 1) / 2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int hcol = hgrp * 16 + lrow;  // query head (within the group) of this lane's column
    const bool hvalid = hcol < p.G;

    // Block-table entries of this split: lane i holds page i of the split.
    const int bt_entry = (lane < n_pages) ? p.bt[(size_t)b * p.maxp + pg_begin + lane] : 0;

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

    char* vst = smem + wave * kWaveLds;  // this wave's V staging: [2 pages][16 tokens][D]
    const size_t head_stride = (size_t)kPage * D;            // elements per (page, head)
    const size_t page_stride = (size_t)p.Hkv * head_stride;  // elements per page

    for (int pair = wave; pair < n_pairs; pair += 4) {
        const int lp0 = 2 * pair, lp1 = 2 * pair + 1;       // local page indexes in the split
        const bool has1 = lp1 < n_pages;
        const int pg0 = __builtin_amdgcn_readlane(bt_entry, lp0);
        const int pg1 = has1 ? __builtin_amdgcn_readlane(bt_entry, lp1) : pg0;
        const uint16_t* kb0 = p.kp + (size_t)pg0 * page_stride + (size_t)g * head_stride;
        const uint16_t* kb1 = p.kp + (size_t)pg1 * page_stride + (size_t)g * head_stride;
        const uint16_t* vb0 = p.vp + (size_t)pg0 * page_stride + (size_t)g * head_stride;
        const uint16_t* vb1 = p.vp + (size_t)pg1 * page_stride + (size_t)g * head_stride;

        // K: A operand, token = lrow, dims 32*ks + 8*lgrp.
        u32x4 kr0[KS], kr1[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kr0[ks] = *reinterpret_cast<const u32x4*>(kb0 + lrow * D + ks * 32 + lgrp * 8);
            kr1[ks] = *reinterpret_cast<const u32x4*>(kb1 + lrow * D + ks * 32 + lgrp * 8);
        }
        // V: whole pages, 16 bytes per lane per load, into LDS row-major.
        constexpr int VL = kPage * D / 8 / 64;  // 16-byte chunks per lane per page
        u32x4 vr0[VL], vr1[VL];
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            vr0[i] = *reinterpret_cast<const u32x4*>(vb0 + (size_t)(i * 64 + lane) * 8);
            vr1[i] = *reinterpret_cast<const u32x4*>(vb1 + (size_t)(i * 64 + lane) * 8);
        }

        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr0[ks]), qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr1[ks]), qf[ks], s1, 0, 0, 0);
        }
        // Mask tokens past the sequence end (and the absent second page).
        const int t0 = tok0 + lp0 * kPage + lgrp * 4;
        const int t1 = tok0 + lp1 * kPage + lgrp * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (t0 + r >= tok1) s0[r] = -INFINITY;
            if (!has1 || t1 + r >= tok1) s1[r] = -INFINITY;
        }
        float m = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                        fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
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
        bf16x8 pf;
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, -ref));
            const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, -ref));
            acc += x0 + x1;
            pf[r] = (__bf16)x0;
            pf[4 + r] = (__bf16)x1;
        }
        lsum += acc;

        // Stage V (row-major, [page][token][D]) and read V^T fragments:
        // A row = dim, k = 8 tokens: tokens 4*lgrp..+3 of page 0 then of page 1.
        // A page that is absent or past the end contributes P = 0, but its V
        // values must still be finite: zero them.
#pragma unroll
        for (int i = 0; i < VL; ++i) {
            *reinterpret_cast<u32x4*>(vst + (i * 64 + lane) * 16) = vr0[i];
            u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(vst + kPage * D * 2 + (i * 64 + lane) * 16) = has1 ? vr1[i] : z;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Tail slots of the last page (tokens >= tok1) may hold any bits,
        // including NaN; 0 * NaN would poison O, so mask them to zero here.
        const uint16_t* vs = reinterpret_cast<const uint16_t*>(vst);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int dim = db * 16 + lrow;
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint16_t x0 = vs[(lgrp * 4 + e) * D + dim];
                uint16_t x1 = vs[kPage * D + (lgrp * 4 + e) * D + dim];
                if (t0 + e >= tok1) x0 = 0;
                if (!has1 || t1 + e >= tok1) x1 = 0;
                a[e] = __builtin_bit_cast(__bf16, x0);
                a[4 + e] = __builtin_bit_cast(__bf16, x1);
            }
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[db], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- merge the 4 waves: (mref, l, O^T) per head column ----
    lsum += xor_lanes(lsum, 16);
    lsum += xor_lanes(lsum, 32);
    __syncthreads();  // V staging is free from here on
    float* st_o = reinterpret_cast<float*>(smem);          // [4 waves][D][16]
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

    const int n_splits = (L + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
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

template <int D>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(DecParams p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long bh = (long long)blockIdx.x * 4 + wave;
    if (bh >= (long long)p.B * p.Hq) return;
    const int b = (int)(bh / p.Hq);
    const int L = p.seq_lens[b];
    const int n = (L + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
    constexpr int DPL = D / 64;  // dims per lane
    if (n == 1) return;          // written by the split kernel
    if (n == 0) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) p.o[bh * D + lane * DPL + e] = 0;
        if (lane == 0) p.lse[bh] = -INFINITY;
        return;
    }
    const float* pl = p.part_lse + bh * p.S;
    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, pl[s]);
    const float Mz = (M == -INFINITY) ? 0.0f : M;
    float den = 0.0f;
    for (int s = 0; s < n; ++s) den += (pl[s] == -INFINITY) ? 0.0f : __expf(pl[s] - Mz);
    const float lse = den > 0.0f ? Mz + logf(den) : -INFINITY;
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
    for (int s = 0; s < n; ++s) {
        const float w = (pl[s] == -INFINITY || den == 0.0f) ? 0.0f : __expf(pl[s] - lse);
        const float* po = p.part_o + ((size_t)bh * p.S + s) * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += w * po[e];
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) p.o[bh * D + lane * DPL + e] = __builtin_bit_cast(uint16_t, (__bf16)acc[e]);
    if (lane == 0) p.lse[bh] = lse;
}

template <int D>
hipError_t launch_t(const DecParams& p, hipStream_t stream) {
    dim3 grid(p.S, p.Hkv * p.n_hgrp, p.B);
    hipLaunchKernelGGL((fa_decode_split_kernel<D>), grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long nbh = (long long)p.B * p.Hq;
    hipLaunchKernelGGL((fa_decode_combine_kernel<D>), dim3((unsigned)((nbh + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

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
    p.S = decode_num_splits(a.max_seq_len);
    p.maxp = a.max_pages_per_seq;
    p.scale_log2 = a.scale * kLog2e;
    p.part_o = static_cast<float*>(a.workspace);
    p.part_lse = p.part_o + (size_t)a.B * a.Hq * p.S * a.d;
    if (a.B == 0) return hipSuccess;
    return a.d == 128 ? launch_t<128>(p, stream) : launch_t<64>(p, stream);
}

}  // namespace fa
