// FP8 (E4M3) attention forward for gfx950, and the block quantizer that
// produces its inputs.
//
// Method (page "FlashAttention" glossary, section "FlashAttention-3": FP8
// support with block quantization): Q, K and V arrive as E4M3 codes with
// float32 scales -- one per 128-row block of Q and of K (a K block is one key
// tile here), one per (batch, K/V head) for V -- and the kernel computes the
// attention equation of the dequantized values, the same IO-aware way as the
// bf16 kernel (tiles streamed through LDS, online softmax in registers, O
// written once):
//   S = (sq * sk_tile * scale) * (Qc Kc^T)      Qc, Kc: codes, product on MFMA
//   P = exp2(S * log2 e - m) <= 2^8             rounded to E4M3 for the PV MFMA
//   O = sv * (sum_tiles P Vc) / l,  LSE = ln 2 * m + ln l
// Both products run on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32
// accumulation; products of codes are exact), twice the bf16 rate and half
// the K/V bytes through HBM and LDS.
//
// gfx950 mapping (same structure as the bf16 kernel in fa_prefill.hip:
// 8 waves of 32 queries sharing a K/V head, scores transposed so a lane
// holds one query, ping-pong of matrix and vector phases across barrier
// slots, lazy rescale with the max-free fast path, XCD-aware grid). What
// changes for FP8:
//   * Staged tiles hold D bytes per row. 16-byte chunks are XOR-swizzled by
//     (row >> 1) & 7 (d = 128) or (row >> 2) & 3 (d = 64), which keeps both
//     read patterns below free of LDS bank conflicts.
//   * K feeds the MFMA A operand (32 bytes = 64 dims per lane) with two
//     16-byte reads; K rows are permuted as in the bf16 kernel, so the score
//     registers of two 32-key blocks are, in order, the 32 key slots of a
//     lane in the PV MFMA's B operand: P is packed to E4M3 in place.
//   * V^T comes from ds_read_b64_tr_b8 (within a 16-lane group, lane i gets
//     byte i%8 of the 8-byte pieces read by lanes 2e + i/8): even and odd
//     lanes read the two 8-dim halves of one key row's chunk, so four such
//     reads give a lane 32 consecutive key slots of one dim.
//   * The next tiles' copies are split unevenly between the wave groups, as
//     in the bf16 kernel but the other way round: here the vector phase is
//     the longer one, so the group that goes on to its vector phase after
//     the barrier copies a quarter of the blocks and the other group three
//     quarters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_kernels.h"
#include "fa_divide.h"
#include "fa_lds.h"

namespace fa {
namespace {

using lds::copy16_to_lds;
using lds::f32x16;
using lds::lds_char;
using lds::max3f;
using lds::other_half;
using lds::row_of_mfma_row;

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBN = 128;        // keys per K/V tile (= one K scale block)
constexpr int kNKB = kBN / 32;  // 32-key blocks per tile
constexpr int kBlockRows = 32;  // queries per row block
constexpr int kBlocksPerWG = 8;
constexpr int kCusPerXcd = 32;
constexpr int kScaleRows = 128;  // rows per Q / K scale block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // P <= 2^8 = 256 < 448, the largest E4M3 value

struct Fp8Params {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    const float* qs;  // [B, Hq, ceil(Nq / 128)]
    const float* ks;  // [B, Hkv, ceil(Nk / 128)]
    const float* vs;  // [B, Hkv]
    uint16_t* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk;
    int G, heads_per_wg, qblocks_per_wg, n_hsub, n_qtiles, n_units, xcd_affine, unit_major;
    int qb_log2;  // log2(qblocks_per_wg)
    FastDiv fd_qtiles, fd_ux, fd_units, fd_hsub, fd_hkv;  // divisions of the workgroup mapping
    float scale_log2;  // softmax scale * log2(e)
};

template <int D>
__device__ __forceinline__ int swz8(int r) {
    if constexpr (D == 128) return (r >> 1) & 7;
    else return (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int toff8(int r, int c) { return r * D + ((c ^ swz8<D>(r)) << 4); }

// Copy rows [j0, j0 + kBN) (clamped to Nk - 1) of a [Nk, D] code matrix into
// a staged tile: 1 KiB per wave instruction.
template <int D>
__device__ __forceinline__ void issue_rows8(const uint8_t* __restrict__ base, lds_char* st, int j0, int Nk, int wave,
                                            int lane) {
    constexpr int RPI = 1024 / D;  // rows per wave instruction
    constexpr int NI = kBN * D / 1024 / kWaves;
    const int uw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int blk = n * kWaves + uw;
        const int r = blk * RPI + lane / (D / 16);
        const int c = (lane % (D / 16)) ^ swz8<D>(r);
        const int key = min(j0 + r, Nk - 1);
        copy16_to_lds(base + (size_t)key * D + c * 16, (uint32_t)(uintptr_t)(st + blk * 1024));
    }
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);  // E4M3 x E4M3, unscaled
}

template <int D>
struct Wave8 {
    static constexpr int KS = D / 64;  // 64-dim k-steps of K Q^T
    static constexpr int DB = D / 32;  // 32-dim blocks of O^T

    i32x8 qf[KS];
    f32x16 oacc[DB];
    float mref, lsum;
    float c;  // this tile's score multiplier in exp2 units: sq * sk * scale * log2 e
    int lim, half, lane;
    int koff[KS][2];  // K A-operand reads (two 16-byte chunks), key block 0
    int voff[DB][4];  // V^T tr_b8 reads, 64-key chunk 0

    __device__ __forceinline__ void mask(f32x16 (&s)[kNKB], int j0) {
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + kb * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                if (key > lim) s[kb][r] = -INFINITY;
            }
    }

    __device__ __forceinline__ void update_ref(const f32x16 (&s)[kNKB]) {
        float m = s[0][0];
#pragma unroll
        for (int i = 1; i + 1 < 16 * kNKB; i += 2)
            m = max3f(m, s[i >> 4][i & 15], s[(i + 1) >> 4][(i + 1) & 15]);
        m = fmaxf(m, s[kNKB - 1][15]);
        m = fmaxf(m, other_half(m));
        const float mx = m * c;
        if (__builtin_amdgcn_ballot_w64(mx > mref + kRescaleSlack) != 0) {
            const float mnew = fmaxf(mref, mx);
            const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mref - mnew);
            mref = mnew;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
    }

    // P = exp2(s * c - ref), packed to E4M3: chunk t (64 keys) holds the
    // registers of key blocks 2t and 2t+1, in order. Returns this lane's
    // share of the tile's row sum.
    __device__ __forceinline__ float probs(const f32x16 (&s)[kNKB], i32x8 (&pf)[kNKB / 2]) {
        const float ref = (mref == -INFINITY) ? 0.0f : mref;
        float acc[4];
#pragma unroll
        for (int t = 0; t < kNKB / 2; ++t)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int kb = 2 * t + (w >> 2);
                const int r0 = (w & 3) * 4;
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r0 + e], c, -ref));
                    acc[e] = (t == 0 && w == 0) ? x[e] : acc[e] + x[e];
                }
                // The two converts write the low and the high half of the
                // register; its previous contents (the last tile's codes)
                // stand in for the half the first one leaves alone, so no
                // zero fill is needed.
                int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], pf[t][w], false);
                v = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
                pf[t][w] = v;
            }
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }

    __device__ __forceinline__ void qk(f32x16 (&s)[kNKB], const lds_char* kst) {
        const f32x16 zero = {};
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int o = kb * 32 * D;
                const i32x4 lo = *reinterpret_cast<const lds_i32x4*>(kst + koff[ks][0] + o);
                const i32x4 hi = *reinterpret_cast<const lds_i32x4*>(kst + koff[ks][1] + o);
                const i32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                s[kb] = mfma8(a, qf[ks], ks == 0 ? zero : s[kb]);
            }
    }

    __device__ __forceinline__ void pv_tile(const i32x8 (&pf)[kNKB / 2], const lds_char* vst) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kNKB / 2; ++t)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                i32x8 a;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_i32x2*)(vst + voff[db][m] + t * 64 * D));
                    a[2 * m] = x[0];
                    a[2 * m + 1] = x[1];
                }
                oacc[db] = mfma8(a, pf[t], oacc[db]);
            }
    }

    // Vector phase. The tile's probabilities are first computed against the
    // current reference without its row max: if no lane's share of the row
    // sum exceeds 2^slack, no P exceeds it either, so the max could not have
    // exceeded the reference by more than the slack and the reference stays
    // (the result is that of always checking the max). Otherwise, and while
    // a row has no reference yet, the max is taken, the reference moved as
    // needed and P recomputed.
    __device__ __forceinline__ void vphase(f32x16 (&s)[kNKB], i32x8 (&pf)[kNKB / 2], int j0, bool masked) {
        __builtin_amdgcn_s_setprio(0);
        if (masked) mask(s, j0);
        constexpr float kSumLimit = 256.0f;  // 2^kRescaleSlack
        float ts = 0.0f;
        bool slow = __builtin_amdgcn_ballot_w64(mref == -INFINITY) != 0;
        if (!slow) {
            ts = probs(s, pf);
            slow = __builtin_amdgcn_ballot_w64(!(ts <= kSumLimit)) != 0;
        }
        if (slow) {
            update_ref(s);
            ts = probs(s, pf);
        }
        lsum += ts;
#pragma unroll
        for (int t = 0; t < kNKB / 2; ++t) asm volatile("" : : "v"(pf[t]));
        asm volatile("" : : "v"(lsum));
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fp8_kernel(Fp8Params p) {
    constexpr int SB = kBN * D;  // bytes of one K or V stage
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * SB];
    lds_char* smem = (lds_char*)smem_raw;
    auto kst = [&](int j) { return smem + (j & 1) * SB; };
    auto vst = [&](int j) { return smem + (2 + (j & 1)) * SB; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int col = lane & 31;

    int unit, qt;
    {
        const int id = blockIdx.x;
        if (p.xcd_affine) {
            const int xcd = id & 7, k = id >> 3;
            const int ux = p.n_units >> 3;
            if (p.unit_major) {
                const int u = fast_div(k, p.fd_qtiles);
                unit = xcd + 8 * u;
                qt = k - u * p.n_qtiles;
            } else {
                qt = fast_div(k, p.fd_ux);
                unit = xcd + 8 * (k - qt * ux);
            }
        } else {
            qt = fast_div(id, p.fd_units);
            unit = id - qt * p.n_units;
        }
        if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest first
    }
    // unit = hsub + n_hsub * (g + Hkv * b)
    const int uh = fast_div(unit, p.fd_hsub);
    const int hsub = unit - uh * p.n_hsub;
    const int b = fast_div(uh, p.fd_hkv);
    const int g = uh - b * p.Hkv;
    const int rows_q = kBlockRows * p.qblocks_per_wg;
    const int qtile0 = qt * rows_q;
    const int Nq = p.Nq, Nk = p.Nk;
    const int head = g * p.G + hsub * p.heads_per_wg + (wave >> p.qb_log2);
    const int q0 = qtile0 + (wave & (p.qblocks_per_wg - 1)) * kBlockRows;
    const int shift = Nk - Nq;

    int wg_kend = Nk, wave_kend = Nk, wave_kmask = Nk;
    if (CAUSAL) {
        const int wg_qlast = min(Nq, qtile0 + rows_q) - 1;
        wg_kend = max(0, min(Nk, wg_qlast + 1 + shift));
        const int wq_last = min(Nq - 1, q0 + kBlockRows - 1);
        wave_kend = max(0, min(Nk, wq_last + 1 + shift));
        wave_kmask = max(0, min(Nk, q0 + 1 + shift));
    }
    if (q0 >= Nq) wave_kend = 0;
    const int n_tiles = (wg_kend + kBN - 1) / kBN;
    const int wt = (wave_kend + kBN - 1) / kBN;
    const int first_masked = wave_kmask / kBN;

    Wave8<D> w;
    {
        const int krow = row_of_mfma_row(col);
#pragma unroll
        for (int ks = 0; ks < Wave8<D>::KS; ++ks)
#pragma unroll
            for (int x = 0; x < 2; ++x) w.koff[ks][x] = toff8<D>(krow, 4 * ks + 2 * half + x);
        // V^T: lane (16q + i): q -> key half kh = q >> 1 and dim half dh = q & 1;
        // i -> key e = i >> 1 of the 8-key run and byte half i & 1.
        const int qg = lane >> 4, i = lane & 15;
        const int kh = qg >> 1, dh = qg & 1, e = i >> 1, odd = i & 1;
#pragma unroll
        for (int db = 0; db < Wave8<D>::DB; ++db)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int row = 16 * m + 8 * kh + e;
                w.voff[db][m] = toff8<D>(row, 2 * db + dh) + 8 * odd;
            }
    }
    w.half = half;
    w.lane = lane;

    // Q codes (B operand: this lane's query, 32 bytes per 64-dim k-step) and
    // the scales.
    const int qi = q0 + col;
    const size_t qrow = ((size_t)b * p.Hq + head) * Nq + min(qi, Nq - 1);
    {
        const uint8_t* qp = p.q + qrow * D;
#pragma unroll
        for (int ks = 0; ks < Wave8<D>::KS; ++ks) {
            const i32x4 lo = *reinterpret_cast<const i32x4*>(qp + ks * 64 + half * 32);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(qp + ks * 64 + half * 32 + 16);
            w.qf[ks] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    }
    const int nqb = (Nq + kScaleRows - 1) / kScaleRows, nkb = (Nk + kScaleRows - 1) / kScaleRows;
    const float sq = p.qs[((size_t)b * p.Hq + head) * nqb + min(q0, Nq - 1) / kScaleRows];
    // K block scales through the constant address space (the kernel never
    // writes them): scalar loads, waited on by lgkmcnt. As ordinary global
    // memory (the copies' asm clobbers memory) each became a vector load whose
    // vmcnt wait also covered the tile copies issued just before it.
    const __attribute__((address_space(4))) float* ksrow =
        (const __attribute__((address_space(4))) float*)(p.ks + ((size_t)b * p.Hkv + g) * nkb);
    const float sqc = sq * p.scale_log2;
    w.lim = CAUSAL ? min(Nk - 1, qi + shift) : Nk - 1;
#pragma unroll
    for (int db = 0; db < Wave8<D>::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.oacc[db][r] = 0.0f;
    w.mref = -INFINITY;
    w.lsum = 0.0f;

    const uint8_t* kbase = p.k + ((size_t)b * p.Hkv + g) * Nk * D;
    const uint8_t* vbase = p.v + ((size_t)b * p.Hkv + g) * Nk * D;
    auto issue_k = [&](int t) { issue_rows8<D>(kbase, kst(t), t * kBN, Nk, wave, lane); };
    auto issue_v = [&](int t) { issue_rows8<D>(vbase, vst(t), t * kBN, Nk, wave, lane); };
    auto set_c = [&](int t) { w.c = sqc * ksrow[t]; };

    if (n_tiles > 0) {
        const bool grp_b = wave >= kWaves / 2;
        issue_k(0);
        issue_v(0);
        if (n_tiles > 1) issue_k(1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        f32x16 s[kNKB];
        i32x8 pf[kNKB / 2] = {};  // defined once; each tile overwrites both halves of every register
        auto end_odd_slot = [&]() {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            asm volatile("s_barrier" ::: "memory");
        };
        // At d = 128 the copies issued after an even barrier are split
        // unevenly between the groups. Group B goes from them into its vector
        // phase, the longer half of each slot here (exponentials and E4M3
        // packing outweigh the FP8 products); group A goes into its matrix
        // phase, which has slack against it. So A's waves copy the V tile
        // (4 of its 16 1 KiB blocks each) and kCopyAK of the K tile's 16
        // blocks each, B's waves the other 4 - kCopyAK K blocks (even
        // split: 2 + 2 each). Measured against the even split: +2.2% with
        // kCopyAK = 2, +2.1% with 4, +1.4% with 0. Block i holds rows
        // 8i..8i+7; a wave's blocks are congruent to it mod 4, hence mod 2,
        // so one lane offset (row in the block, swizzled chunk) serves all.
        constexpr int kCopyAK = 2;
        const int cp_row = lane / (D / 16);
        const int cp_col = ((lane % (D / 16)) ^ swz8<D>(8 * (wave & 1) + cp_row)) * 16;
        auto issue_blocks = [&](const uint8_t* base, lds_char* st, int j0, int first, auto count) {
            constexpr int RPI = 1024 / D;  // rows per block
            const int uf = __builtin_amdgcn_readfirstlane(first);
#pragma unroll
            for (int m = 0; m < decltype(count)::value; ++m) {
                const int blk = uf + 4 * m;
                const int key = min(j0 + blk * RPI + cp_row, Nk - 1);
                copy16_to_lds(base + (size_t)key * D + cp_col, (uint32_t)(uintptr_t)(st + blk * 1024));
            }
        };
        // copies for slot 2j+1 landed; issue the next ones (group B: is_b)
        auto end_even_slot = [&](int j, auto is_b) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if constexpr (D != 128) {
                if (j + 2 < n_tiles) issue_k(j + 2);
                if (j + 1 < n_tiles) issue_v(j + 1);
            } else {
                const int uw = wave & 3;
                if constexpr (!decltype(is_b)::value) {
                    if (j + 1 < n_tiles) issue_blocks(vbase, vst(j + 1), (j + 1) * kBN, uw, std::integral_constant<int, 4>{});
                    if (j + 2 < n_tiles)
                        issue_blocks(kbase, kst(j + 2), (j + 2) * kBN, uw, std::integral_constant<int, kCopyAK>{});
                } else {
                    if (j + 2 < n_tiles)
                        issue_blocks(kbase, kst(j + 2), (j + 2) * kBN, 4 * kCopyAK + uw,
                                     std::integral_constant<int, 4 - kCopyAK>{});
                }
            }
        };
        int j = 0;
        if (!grp_b) {
            if (wt > 0) w.qk(s, kst(0));
            for (; j + 1 < wt; ++j) {
                if (j > 0) end_odd_slot();
                set_c(j);
                w.vphase(s, pf, j * kBN, j >= first_masked);
                end_even_slot(j, std::false_type{});
                w.pv_tile(pf, vst(j));
                w.qk(s, kst(j + 1));
            }
            if (j < wt) {
                if (j > 0) end_odd_slot();
                set_c(j);
                w.vphase(s, pf, j * kBN, j >= first_masked);
                end_even_slot(j, std::false_type{});
                w.pv_tile(pf, vst(j));
                ++j;
            }
            for (;; ++j) {
                if (j > 0) end_odd_slot();
                if (j == n_tiles) break;
                end_even_slot(j, std::false_type{});
            }
        } else {
            if (wt > 0) w.qk(s, kst(0));
            end_even_slot(0, std::true_type{});
            if (wt > 0) {
                set_c(0);
                w.vphase(s, pf, 0, 0 >= first_masked);
            }
            for (j = 1; j < wt; ++j) {
                end_odd_slot();
                w.pv_tile(pf, vst(j - 1));
                w.qk(s, kst(j));
                end_even_slot(j, std::true_type{});
                set_c(j);
                w.vphase(s, pf, j * kBN, j >= first_masked);
            }
            bool done = false;
            if (wt > 0) {
                end_odd_slot();
                w.pv_tile(pf, vst(j - 1));
                if (j == n_tiles) done = true;
                else end_even_slot(j++, std::true_type{});
            }
            if (!done)
                for (;; ++j) {
                    end_odd_slot();
                    if (j == n_tiles) break;
                    end_even_slot(j, std::true_type{});
                }
        }
    }
    __builtin_amdgcn_s_setprio(0);

    // O = sv * O^T / l (transposed back on store), LSE = ln 2 * m + ln l.
    const float l = w.lsum + other_half(w.lsum);
    const float inv = l > 0.0f ? p.vs[(size_t)b * p.Hkv + g] / l : 0.0f;
    if (qi < Nq) {
        uint16_t* op = p.o + qrow * D;
#pragma unroll
        for (int db = 0; db < Wave8<D>::DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(w.oacc[db][r4 * 4 + e] * inv);
                *reinterpret_cast<bf16x4*>(op + db * 32 + r4 * 8 + half * 4) = ov;
            }
        if (half == 0) p.lse[qrow] = l > 0.0f ? (w.mref * kLn2 + logf(l)) : -INFINITY;
    }
}

// ---- block quantizer ---------------------------------------------------------
// One workgroup per (batch, head, block of `block_rows` rows): the block's
// largest magnitude, then scale = amax / 448 (1 for an all-zero block) and
// codes = E4M3(x / scale), each computed in float32 (correctly rounded
// quotient, round-to-nearest-even conversion). A block of up to 8 x 2048
// elements (128 rows at d = 128) keeps its loads in registers between the two
// steps; longer ones (V's one block per head) read x twice.
//
// The quotient: with r = 1 / scale rounded once, q = x r followed by two
// residual corrections q += (x - scale q) r (fma) is the correctly rounded
// quotient (Markstein's theorem: r within half an ulp of 1 / scale, q within
// an ulp after the first correction), as long as the residuals do not
// underflow. That holds for scale >= 2^-60 wherever the quotient is at least
// 2^-12; below that its E4M3 code is 0 either way. Smaller scales take the
// division instruction sequence.
__device__ __forceinline__ float quotient_fast(float x, float sc, float rc) {
    float q = x * rc;
    q = __builtin_fmaf(__builtin_fmaf(-sc, q, x), rc, q);
    return __builtin_fmaf(__builtin_fmaf(-sc, q, x), rc, q);
}

template <bool kFastDiv>
__device__ __forceinline__ i32x2 quantize8(const i32x4 v, float sc, float rc) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t u = (uint32_t)v[e];
        f[2 * e] = __uint_as_float(u << 16);
        f[2 * e + 1] = __uint_as_float(u & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = kFastDiv ? quotient_fast(f[e], sc, rc) : f[e] / sc;
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    return i32x2{lo, hi};
}

__device__ __forceinline__ float amax8(const i32x4 v, float amax) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t u = (uint32_t)v[e];
        amax = fmaxf(amax, fabsf(__uint_as_float(u << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(u & 0xffff0000u)));
    }
    return amax;
}

__global__ __launch_bounds__(256) void fa_quantize_fp8_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales, int N, int d,
                                                             int block_rows, int nb) {
    constexpr int kStep = 256 * 8;  // elements per pass of the workgroup
    constexpr int kHeld = 8;        // passes kept in registers
    const int blk = blockIdx.x % nb;
    const size_t bh = blockIdx.x / nb;
    const int r0 = blk * block_rows, r1 = min(N, r0 + block_rows);
    const size_t base = (bh * N + r0) * (size_t)d;
    const size_t n = (size_t)(r1 - r0) * d;  // a multiple of 8 (d is 64 or 128)
    const size_t i0 = (size_t)threadIdx.x * 8;
    __shared__ float wmax[4];
    auto block_scale = [&](float amax) {
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        if (threadIdx.x == 0) scales[blockIdx.x] = sc;
        return sc;
    };
    if (n <= (size_t)kHeld * kStep) {
        i32x4 v[kHeld];
#pragma unroll
        for (int m = 0; m < kHeld; ++m)
            if (i0 + m * kStep < n) v[m] = *reinterpret_cast<const i32x4*>(x + base + i0 + m * kStep);
        float amax = 0.0f;
#pragma unroll
        for (int m = 0; m < kHeld; ++m)
            if (i0 + m * kStep < n) amax = amax8(v[m], amax);
        const float sc = block_scale(amax);
        const float rc = 1.0f / sc;
        if (sc >= 0x1p-60f) {
#pragma unroll
            for (int m = 0; m < kHeld; ++m)
                if (i0 + m * kStep < n)
                    *reinterpret_cast<i32x2*>(codes + base + i0 + m * kStep) = quantize8<true>(v[m], sc, rc);
        } else {
#pragma unroll
            for (int m = 0; m < kHeld; ++m)
                if (i0 + m * kStep < n)
                    *reinterpret_cast<i32x2*>(codes + base + i0 + m * kStep) = quantize8<false>(v[m], sc, rc);
        }
        return;
    }
    float amax = 0.0f;
    for (size_t i = i0; i < n; i += kStep) amax = amax8(*reinterpret_cast<const i32x4*>(x + base + i), amax);
    const float sc = block_scale(amax);
    const float rc = 1.0f / sc;
    for (size_t i = i0; i < n; i += kStep) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(x + base + i);
        *reinterpret_cast<i32x2*>(codes + base + i) =
            sc >= 0x1p-60f ? quantize8<true>(v, sc, rc) : quantize8<false>(v, sc, rc);
    }
}

// ---- incoherent processing, then the block quantizer ---------------------------
// Each row is first multiplied by M = diag(s) H_d / sqrt(d) (s: the caller's
// signs, H_d: Sylvester's Hadamard matrix, H[i][j] = (-1)^popcount(i & j)).
// M is orthogonal, so Q and K transformed with the same signs keep Q K^T, and
// a large entry is spread over all d channels before it sets its block's
// scale. Then, as above, scale = amax / 448 and codes = E4M3(y / scale) in
// float32.
//
// A lane holds 32 consecutive channels of a row (D / 32 lanes per row, so 4
// or 2 lanes: a row never leaves its quad). The fast Walsh-Hadamard
// transform's butterflies (y_j, y_j+h) <- (y_j + y_j+h, y_j - y_j+h) with
// stride h < 32 run in registers; strides 32 and 64 pair lanes that differ in
// one bit of their index within the row, exchanged by DPP quad permutes
// (new = partner + (+-1) * own, one fma that rounds once, like the add or
// subtract it stands for). The signs are applied by flipping sign bits and
// the 1 / sqrt(d) comes last. A block of up to two passes of the workgroup
// (128 rows at d = 128, 256 at d = 64) stays in registers between its
// largest magnitude and its codes; longer blocks transform twice, in the same
// instructions, so the element that sets the scale lands on +-448 either way.
// The quotient y / scale is computed as in the block quantizer above.
constexpr int kIncLanesChannels = 32;   // channels per lane

struct IncLoad {
    i32x4 v[4];
};

__device__ __forceinline__ IncLoad inc_load(const uint16_t* __restrict__ src) {
    IncLoad l;
#pragma unroll
    for (int c = 0; c < 4; ++c) l.v[c] = *reinterpret_cast<const i32x4*>(src + c * 8);
    return l;
}

template <int D>
__device__ __forceinline__ void incoherent_row32(const IncLoad& l, const uint32_t (&flip)[32], float (&f)[32]) {
    constexpr float kNorm = D == 64 ? 0.125f : 0.08838834764831845f;  // 1 / sqrt(D), rounded once
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t u = (uint32_t)l.v[c][e];
            f[c * 8 + 2 * e] = __uint_as_float((u << 16) ^ flip[c * 8 + 2 * e]);
            f[c * 8 + 2 * e + 1] = __uint_as_float((u & 0xffff0000u) ^ flip[c * 8 + 2 * e + 1]);
        }
#pragma unroll
    for (int h = 1; h < kIncLanesChannels; h <<= 1)
#pragma unroll
        for (int j = 0; j < kIncLanesChannels; ++j)
            if ((j & h) == 0) {
                const float a = f[j], b = f[j + h];
                f[j] = a + b;
                f[j + h] = a - b;
            }
    // Strides 32 (lane bit 0) and, for D = 128, 64 (lane bit 1): the lower
    // lane keeps a + b, the upper one a - b, where a is the lower lane's value.
    const int lr = threadIdx.x % (D / kIncLanesChannels);
#pragma unroll
    for (int m = 1; m < D / kIncLanesChannels; m <<= 1) {
        const float own = (lr & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < kIncLanesChannels; ++j) {
            const int other = m == 1 ? __builtin_amdgcn_mov_dpp(__float_as_int(f[j]), 0xB1, 0xF, 0xF, false)  // [1,0,3,2]
                                     : __builtin_amdgcn_mov_dpp(__float_as_int(f[j]), 0x4E, 0xF, 0xF, false); // [2,3,0,1]
            f[j] = __builtin_fmaf(own, f[j], __int_as_float(other));
        }
    }
#pragma unroll
    for (int j = 0; j < kIncLanesChannels; ++j) f[j] *= kNorm;
}

// E4M3 codes of f[] / sc for 32 channels, stored at dst (32 bytes).
template <bool kFastDiv>
__device__ __forceinline__ void inc_store_codes(const float (&f)[32], float sc, float rc, uint8_t* __restrict__ dst) {
    float t[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        t[j] = kFastDiv ? quotient_fast(f[j], sc, rc) : f[j] / sc;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        int w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float* g = t + c * 16 + e * 4;
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(g[0], g[1], 0, false);
            w[e] = __builtin_amdgcn_cvt_pk_fp8_f32(g[2], g[3], lo, true);
        }
        *reinterpret_cast<i32x4*>(dst + c * 16) = i32x4{w[0], w[1], w[2], w[3]};
    }
}

template <int D>
__global__ __launch_bounds__(256) void fa_quantize_fp8_incoherent_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ signs, uint8_t* __restrict__ codes,
    float* __restrict__ scales, int N, int block_rows, int nb) {
    constexpr int kStep = 256 * kIncLanesChannels;  // elements per pass of the workgroup (a multiple of D)
    const int blk = blockIdx.x % nb;
    const size_t bh = blockIdx.x / nb;
    const int r0 = blk * block_rows, r1 = min(N, r0 + block_rows);
    const size_t base = (bh * N + r0) * (size_t)D;
    const size_t n = (size_t)(r1 - r0) * D;  // whole rows, so the lanes of a row are active together
    const size_t i0 = (size_t)threadIdx.x * kIncLanesChannels;
    const int c0 = (threadIdx.x % (D / kIncLanesChannels)) * kIncLanesChannels;
    uint32_t flip[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) flip[j] = signs[c0 + j] < 0 ? 0x80000000u : 0u;
    __shared__ float wmax[4];
    auto block_scale = [&](float amax) {
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        if (threadIdx.x == 0) scales[blockIdx.x] = sc;
        return sc;
    };
    if (n <= 2 * (size_t)kStep) {
        // the whole block in registers: every load first, then the transforms
        const bool have0 = i0 < n, have1 = i0 + kStep < n;
        IncLoad l0, l1;
        if (have0) l0 = inc_load(x + base + i0);
        if (have1) l1 = inc_load(x + base + i0 + kStep);
        float f0[32], f1[32];
        float amax = 0.0f;
        if (have0) {
            incoherent_row32<D>(l0, flip, f0);
#pragma unroll
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f0[j]));
        }
        if (have1) {
            incoherent_row32<D>(l1, flip, f1);
#pragma unroll
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f1[j]));
        }
        const float sc = block_scale(amax);
        const float rc = 1.0f / sc;
        if (sc >= 0x1p-60f) {
            if (have0) inc_store_codes<true>(f0, sc, rc, codes + base + i0);
            if (have1) inc_store_codes<true>(f1, sc, rc, codes + base + i0 + kStep);
        } else {
            if (have0) inc_store_codes<false>(f0, sc, rc, codes + base + i0);
            if (have1) inc_store_codes<false>(f1, sc, rc, codes + base + i0 + kStep);
        }
        return;
    }
    float amax = 0.0f;
    for (size_t i = i0; i < n; i += kStep) {
        float f[32];
        incoherent_row32<D>(inc_load(x + base + i), flip, f);
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f[j]));
    }
    const float sc = block_scale(amax);
    const float rc = 1.0f / sc;
    for (size_t i = i0; i < n; i += kStep) {
        float f[32];
        incoherent_row32<D>(inc_load(x + base + i), flip, f);
        if (sc >= 0x1p-60f) inc_store_codes<true>(f, sc, rc, codes + base + i);
        else inc_store_codes<false>(f, sc, rc, codes + base + i);
    }
}

int pow2_divisor_upto8(int G) {
    int h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

}  // namespace

hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream) {
    Fp8Params p = {};
    p.q = static_cast<const uint8_t*>(a.q);
    p.k = static_cast<const uint8_t*>(a.k);
    p.v = static_cast<const uint8_t*>(a.v);
    p.qs = a.q_scales;
    p.ks = a.k_scales;
    p.vs = a.v_scales;
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
    p.G = a.Hq / a.Hkv;
    p.heads_per_wg = pow2_divisor_upto8(p.G);
    p.qblocks_per_wg = kBlocksPerWG / p.heads_per_wg;
    p.n_hsub = p.G / p.heads_per_wg;
    p.n_qtiles = (a.Nq + kBlockRows * p.qblocks_per_wg - 1) / (kBlockRows * p.qblocks_per_wg);
    p.n_units = a.B * a.Hkv * p.n_hsub;
    p.xcd_affine = (p.n_units % 8 == 0) ? 1 : 0;
    p.unit_major = (p.n_qtiles >= kCusPerXcd) ? 1 : 0;
    p.qb_log2 = 0;
    while ((1 << p.qb_log2) < p.qblocks_per_wg) ++p.qb_log2;
    p.fd_qtiles = make_fastdiv(p.n_qtiles);
    p.fd_ux = make_fastdiv(p.n_units >= 8 ? p.n_units >> 3 : 1);
    p.fd_units = make_fastdiv(p.n_units);
    p.fd_hsub = make_fastdiv(p.n_hsub);
    p.fd_hkv = make_fastdiv(a.Hkv);
    p.scale_log2 = a.scale * kLog2e;
    const long long grid = (long long)p.n_units * p.n_qtiles;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_on())
        trace("fa_fwd_fp8_kernel<d=%d, causal=%d> grid=%lld block=%d (units=%d x query tiles=%d)", a.d,
              a.causal ? 1 : 0, grid, kThreads, p.n_units, p.n_qtiles);
    if (a.d == 128) {
        if (a.causal) hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, true>), dim3((int)grid), dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, false>), dim3((int)grid), dim3(kThreads), 0, stream, p);
    } else {
        if (a.causal) hipLaunchKernelGGL((fa_fwd_fp8_kernel<64, true>), dim3((int)grid), dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((fa_fwd_fp8_kernel<64, false>), dim3((int)grid), dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, void* codes, float* scales, int B, int H, int N, int d, int block_rows,
                               hipStream_t stream) {
    const long long nb = (N + block_rows - 1) / block_rows;
    const long long grid = (long long)B * H * nb;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_on()) trace("fa_quantize_fp8_kernel grid=%lld block=256 (block_rows=%d)", (long long)grid, block_rows);
    hipLaunchKernelGGL(fa_quantize_fp8_kernel, dim3((int)grid), dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       static_cast<uint8_t*>(codes), scales, N, d, block_rows, (int)nb);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8_incoherent(const void* x, const int8_t* signs, void* codes, float* scales, int B, int H,
                                          int N, int d, int block_rows, hipStream_t stream) {
    const long long nb = (N + block_rows - 1) / block_rows;
    const long long grid = (long long)B * H * nb;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_on())
        trace("fa_quantize_fp8_incoherent_kernel<d=%d> grid=%lld block=256 (block_rows=%d)", d, (long long)grid,
              block_rows);
    if (d == 128)
        hipLaunchKernelGGL(fa_quantize_fp8_incoherent_kernel<128>, dim3((int)grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), signs, static_cast<uint8_t*>(codes), scales, N, block_rows,
                           (int)nb);
    else
        hipLaunchKernelGGL(fa_quantize_fp8_incoherent_kernel<64>, dim3((int)grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), signs, static_cast<uint8_t*>(codes), scales, N, block_rows,
                           (int)nb);
    return hipGetLastError();
}

}  // namespace fa
