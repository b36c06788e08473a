// Prefill attention forward for gfx950 (CDNA4): O = softmax(scale*Q K^T + mask) V.
//
// Method (pages: "FlashAttention" glossary, section "L'idee cle :
// IO-awareness"; "Comment Flash Attention reduit-il le trafic memoire ...",
// sections on tiles, the online softmax and kernel fusion): K/V are streamed
// in tiles through on-chip memory, scores stay in registers, and a running
// row max / row sum are rescaled so the result is exact. Scores, scaling, the
// causal mask, the softmax and the product with V are fused in this one
// kernel; O is written once.
//
// gfx950 mapping (this file's own design):
//   * Workgroup = 8 waves = 8 row blocks of 32 queries, one block per wave,
//     two waves per SIMD (waves w and w+4 share one). A row block is 32
//     consecutive queries of one query head. The 8 blocks of a workgroup
//     share one K/V head (GQA packing): for a group size G they are
//     min(G, 8) heads x (8 / min(G, 8)) query blocks.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 result each lane holds one query
//     (column) and 16 keys (rows), so the softmax max / sum are in-lane
//     reductions plus one exchange between the two 32-lane halves.
//   * The K rows fed to the MFMA are permuted so that result register r of
//     lane half h holds key 16*(r/8) + 8*h + r%8 of the 32-key block. The
//     exponentiated scores then already form the B operand of the second MFMA,
//     O^T += V^T P^T, with keys in natural order -- no data movement.
//   * K and V tiles go from global memory straight into LDS
//     (global_load_lds_dwordx4, no registers involved), row-major with an XOR
//     swizzle of 16-byte chunks. K feeds the MFMA A operand with 16-byte LDS
//     reads; V^T fragments come from the gfx950 transposing LDS read
//     ds_read_b64_tr_b16 (within a 16-lane group, lane i receives element
//     i%4 of the 8-byte pieces read by lanes 4e + i/4, e = 0..3), so V is
//     never transposed in registers. The swizzle keeps both read patterns
//     free of bank conflicts. K and V each have two LDS stages.
//   * Ping-pong: the two waves of a SIMD run half a tile apart. Workgroup
//     barriers cut time into slots; in every slot one wave of each SIMD runs
//     its matrix phase (PV product of one tile, then the scores of the next)
//     while the other runs its vector phase (mask, max, exponentials, sums).
//     A single barrier per tile would instead keep both waves in the same
//     phase, leaving the matrix cores idle during every softmax.
//   * The next tiles' copies are issued right after the barrier that ends a
//     vector phase of the leading group. That group goes on to its matrix
//     phase, which is on the tile's critical path; the other group goes on
//     to its vector phase, which has slack. So the copies are split unevenly
//     (d = 128, contiguous or paged K/V): the leading group copies a quarter,
//     the other three quarters, full tiles from scalar bases.
//   * LDS read offsets are kept as one base per read kind; the k-step and
//     dim-block offsets differ from it by an xor with a constant, which
//     frees the registers a table of offsets would hold.
//   * Lazy rescaling: the running maximum used as the softmax reference is
//     only moved when some row's tile maximum exceeds it by more than 2^8 in
//     exp2 units. The reference cancels exactly between O and the row sum, so
//     the result is unchanged while most tiles skip the O rescale. Most tiles
//     also skip the row max itself: P is first computed against the current
//     reference, and the max is only taken (and P recomputed) when some
//     lane's share of the tile's row sum exceeds 2^8, which any move of the
//     reference would imply.
//   * Built without NaN semantics (-fno-honor-nans): the row max of MFMA
//     results then needs no NaN-quieting instructions. Nothing here relies
//     on NaN: masked scores are -inf, and every path keeps -inf out of
//     inf - inf (the reference is replaced by 0 while it is -inf).
//   * Grid: one workgroup per (batch, K/V head, head subset, query tile).
//     Query tiles are issued heaviest-first for causal masks, and when there
//     are a multiple of 8 K/V units, all tiles of one K/V head go to one XCD
//     (workgroups are dealt round-robin to the 8 XCDs) so they share its L2.
//     When a unit has at least 32 query tiles (one XCD's CUs), an XCD runs
//     one unit's tiles at a time, so its L2 holds one unit's K/V.
//   * Paged mode (chunked prefill): the same kernel reads K/V pages through
//     the page table; each copy instruction's page id is loaded one tile
//     ahead. Query rows are packed per sequence (token-major).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_kernels.h"
#include "fa_divide.h"
#include "fa_lds.h"

namespace fa {
namespace {

using namespace lds;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
#ifndef FA_PREFILL_BN
#define FA_PREFILL_BN 128
#endif
constexpr int kBN = FA_PREFILL_BN;  // keys per K/V tile
constexpr int kNKB = kBN / 32;      // 32-key blocks per tile
constexpr int kBlockRows = 32;      // queries per row block
constexpr int kBlocksPerWG = 8;
constexpr int kCusPerXcd = 32;      // MI355X: 256 CUs in 8 XCDs
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // exp2 units the reference may lag behind the max
constexpr int kLdsLead = 4;            // LDS fragment reads issued this many MFMAs ahead
// Block-sparse mode: mask blocks are 128 queries x 128 keys (one K/V tile);
// a workgroup's list of active key tiles lives in LDS after the K/V stages.
constexpr int kSparseBlock = kSparseMaskBlock;
constexpr int kMaxSparseTiles = kSparseMaxKeyBlocks;
constexpr int kSparseLdsBytes = (kMaxSparseTiles + 1 + 8) * 4;
constexpr int kNoKey = 1 << 30;        // tile start that masks every key of a tile

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, Hq, Hkv, Nq, Nk;
    int G;               // query heads per K/V head
    int heads_per_wg;    // largest power of two <= 8 dividing G
    int qblocks_per_wg;  // 8 / heads_per_wg
    int n_hsub;          // G / heads_per_wg
    int n_qtiles;        // ceil(Nq / (32 * qblocks_per_wg))
    int n_units;         // B * Hkv * n_hsub
    int xcd_affine;      // n_units % 8 == 0
    int unit_major;      // n_qtiles >= CUs per XCD: an XCD runs one unit's tiles at a time
    int qb_log2;         // log2(qblocks_per_wg)
    // Divisions of the workgroup mapping: by n_qtiles, n_units / 8, n_units,
    // n_hsub and Hkv.
    FastDiv fd_qtiles, fd_ux, fd_units, fd_hsub, fd_hkv;
    int causal;
    float scale_log2;    // scale * log2(e)
    float scale;
    // Sliding window, in key positions relative to the query's bottom-right
    // aligned position p = i + Nk - Nq: keys below p - win_left are masked
    // (win_left < 0: none); with a right bound (the CAUSAL instantiation),
    // keys above p + win_right are masked (0 for plain causal).
    int win_left, win_right;
    // Paged mode only: per-sequence lengths and the page table.
    const int32_t* bt;        // [B, maxp] page ids
    const int32_t* seq_lens;  // [B] context length (keys) of each sequence
    const int32_t* cu_q;      // [B + 1] first packed query row of each sequence
    int maxp;
    // Block-sparse mode only: mask [B, Hq, ceil(Nq/128), n_kb] bytes with
    // batch / head strides bm_sb / bm_sh (0 broadcasts).
    const uint8_t* bmask;
    long long bm_sb, bm_sh;
    int n_kb;
};

template <int D>
struct Stage {
    static constexpr int kBytesK = kBN * D * 2;
    static constexpr int kInstPerWave = kBytesK / 1024 / kWaves;  // 1 KiB per wave instruction
};

// Enqueue the direct global->LDS copy of rows [j0, j0 + kBN) of one K or V
// tile into a stage. Rows past Nk are clamped to the last row: they are
// masked out of the scores (K) and meet zero weights (V), and stay finite.
// Each wave instruction copies 1 KiB = RPI aligned rows (4 at d=128, 8 at
// d=64), which never straddle a 16-row page.
//   Contiguous (pg == nullptr): row `key` is at base + key * D.
//   Paged: pg[n] is the page holding instruction n's rows (page_ids());
//   base is the pool at K/V head g, row `key` is at slot key % 16.
template <int D>
__device__ __forceinline__ void issue_rows(const uint16_t* __restrict__ base, const int* pg, size_t page_stride,
                                           lds_char* st, int j0, int Nk, int wave, int lane) {
    constexpr int RB = D * 2;          // bytes per row
    constexpr int RPI = 1024 / RB;     // rows per wave instruction
    static_assert(16 % RPI == 0, "copy rows must not straddle a page");
    const int uw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int n = 0; n < Stage<D>::kInstPerWave; ++n) {
        const int blk = n * kWaves + uw;              // which 1 KiB of the tile
        const int r = blk * RPI + lane / (RB / 16);
        const int phys = lane % (RB / 16);
        const int c = phys ^ swz<D>(r);
        const int key = min(j0 + r, Nk - 1);
        const uint16_t* row = pg ? base + (size_t)pg[n] * page_stride + (size_t)(key & 15) * D
                                 : base + (size_t)key * D;
        copy16_to_lds(row + c * 8, (uint32_t)(uintptr_t)(st + blk * 1024));
    }
}

// Page ids of the rows issue_rows() copies for the tile at key offset j0
// (one table entry per copy instruction), loaded a slot ahead of the copies.
// The table is read through the constant address space: the kernel never
// writes it, so the compiler may use scalar loads (waited on by lgkmcnt)
// although the copies' asm clobbers memory. Otherwise it reads the entry
// with a vector load and waits on vmcnt right away to move it to an SGPR --
// and vmcnt also counts the tile copies just issued, so every issue point
// waited for them to land (measured: 12.7% of the paged prefill's time).
template <int D>
__device__ __forceinline__ void page_ids(int (&pg)[Stage<D>::kInstPerWave], const int32_t* bt_row, int j0, int Nk,
                                         int wave) {
    constexpr int RPI = 1024 / (D * 2);
    const int uw = __builtin_amdgcn_readfirstlane(wave);
    const __attribute__((address_space(4))) int32_t* cbt = (const __attribute__((address_space(4))) int32_t*)bt_row;
#pragma unroll
    for (int n = 0; n < Stage<D>::kInstPerWave; ++n) {
        const int first = min(j0 + (n * kWaves + uw) * RPI, Nk - 1);
        pg[n] = cbt[first >> 4];
    }
}

// Page ids for the uneven copy split: ids[m] is the page holding rows
// j0 + 16 (m0 + m) .. +15 of a tile, clamped to the page of the last key.
template <int N>
__device__ __forceinline__ void page_ids_run(int (&ids)[N], const int32_t* bt_row, int j0, int m0, int Nk) {
    const __attribute__((address_space(4))) int32_t* cbt = (const __attribute__((address_space(4))) int32_t*)bt_row;
    const int last = (Nk - 1) >> 4;
#pragma unroll
    for (int m = 0; m < N; ++m) ids[m] = cbt[min((j0 >> 4) + m0 + m, last)];
}

// Per-wave state (one row block) and its matrix / vector phases.
template <int D>
struct Wave {
    static constexpr int KS = D / 16;   // 16-dim k-steps of K Q^T
    static constexpr int DB = D / 32;   // 32-dim blocks of O^T

    bf16x8 qf[KS];
    f32x16 oacc[DB];
    float mref;  // reference max, in exp2 units (score * scale_log2)
    float lsum;  // this lane half's share of the row sum
    int lim, lo, half, lane;  // visible keys of this lane's query: [lo, lim]
    // LDS byte offsets of this lane's reads, kept as one base each: the K
    // fragment of k-step ks (key block 0; block kb adds 32 rows) is at
    // koff0 ^ (ks << 5), the V^T reads of dim block db (16-key slice 0) at
    // voff0[h] ^ (db << 6) (see tile_off_ks / tr_off_db).
    int koff0;
    int voff0[2];
    float scale_log2;

    // WIN: the lower (window) edge is masked as well.
    template <bool WIN>
    __device__ __forceinline__ void mask(f32x16 (&s)[kNKB], int j0) {
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + kb * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                if (key > lim || (WIN && key < lo)) s[kb][r] = -INFINITY;
            }
    }

    // Row max of a tile's scores; moves the reference (and rescales O and
    // the row sum) only when some row's max exceeds it by more than the slack.
    __device__ __forceinline__ void update_ref(const f32x16 (&s)[kNKB]) {
        float m = s[0][0];
#pragma unroll
        for (int i = 1; i + 1 < 16 * kNKB; i += 2)
            m = max3f(m, s[i >> 4][i & 15], s[(i + 1) >> 4][(i + 1) & 15]);
        m = fmaxf(m, s[kNKB - 1][15]);
        m = fmaxf(m, other_half(m));
        const float mx = m * scale_log2;
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

    // P = exp2(s * scale_log2 - ref) in bf16, the B operand of the PV product.
    // Returns this lane's share of the tile's row sum.
    __device__ __forceinline__ float probs(const f32x16 (&s)[kNKB], bf16x8 (&pf)[2 * kNKB]) {
        const float ref = (mref == -INFINITY) ? 0.0f : mref;
        float acc[4];  // independent partial sums (short add chains), started by the first four values
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                bf16x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][h8 * 8 + e], scale_log2, -ref));
                    acc[e & 3] = (kb == 0 && h8 == 0 && e < 4) ? x : acc[e & 3] + x;
                    pv[e] = (__bf16)x;
                }
                pf[kb * 2 + h8] = pv;
            }
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }

    // Scores of a staged K tile; each K fragment is read kLdsLead MFMAs ahead.
    __device__ __forceinline__ void qk(f32x16 (&s)[kNKB], const lds_char* kst) {
        constexpr int NQ = KS * kNKB;
        u32x4 kf[KS][kNKB];
        // The per-k-step offsets are derived here on every call, not kept
        // across the loop (the empty asm makes the base opaque, so the
        // compiler cannot hoist them): 7 registers fewer in the loop, at no
        // extra instruction (the xor folds into the address add).
        int k0 = koff0;
        asm volatile("" : "+v"(k0));
        auto kread = [&](int n) {
            kf[n / kNKB][n % kNKB] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                kst + tile_off_ks(k0, n / kNKB) + (n % kNKB) * 32 * (D * 2));
        };
        const f32x16 zero = {};
#pragma unroll
        for (int n = 0; n < kLdsLead && n < NQ; ++n) kread(n);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            if (n + kLdsLead < NQ) kread(n + kLdsLead);
            const int ks = n / kNKB, kb = n % kNKB;
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ks][kb]), qf[ks], ks == 0 ? zero : s[kb],
                                                           0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // O^T += V^T P^T for a staged V tile; V^T fragments read kLdsLead MFMAs ahead.
    __device__ __forceinline__ void pv_tile(const bf16x8 (&pf)[2 * kNKB], const lds_char* vst) {
        // The matrix phase gets issue priority over the partner wave's
        // softmax on the same SIMD (reset when the vector phase starts).
        __builtin_amdgcn_s_setprio(1);
        constexpr int NP = 2 * kNKB * DB;
        bf16x8 vf[2 * kNKB][DB];
        int v0[2] = {voff0[0], voff0[1]};  // opaque bases, as in qk()
        asm volatile("" : "+v"(v0[0]), "+v"(v0[1]));
        auto vread = [&](int n) { vf[n / DB][n % DB] = read_tr_db<D>(vst, v0, n % DB, n / DB); };
#pragma unroll
        for (int n = 0; n < kLdsLead && n < NP; ++n) vread(n);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            if (n + kLdsLead < NP) vread(n + kLdsLead);
            const int t = n / DB, db = n % DB;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][db], pf[t], oacc[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // pv_tile(pf, vst) then qk(s, kst) as one stream of MFMAs: the LDS reads
    // run kLdsLead products ahead across the boundary, so the first score
    // product does not wait for its K fragment (measured +0.5% on the 8K
    // causal GQA prefill, +2% on the 2K MHA one).
    __device__ __forceinline__ void pv_qk(const bf16x8 (&pf)[2 * kNKB], const lds_char* vst, f32x16 (&s)[kNKB],
                                          const lds_char* kst) {
        __builtin_amdgcn_s_setprio(1);
        constexpr int NP = 2 * kNKB * DB;
        constexpr int NQ = KS * kNKB;
        bf16x8 buf[NP + NQ];
        int v0[2] = {voff0[0], voff0[1]};
        asm volatile("" : "+v"(v0[0]), "+v"(v0[1]));
        int k0 = koff0;
        asm volatile("" : "+v"(k0));
        auto rd = [&](int n) {
            if (n < NP) {
                buf[n] = read_tr_db<D>(vst, v0, n % DB, n / DB);
            } else {
                const int m = n - NP;
                buf[n] = as_bf16x8(*reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                    kst + tile_off_ks(k0, m / kNKB) + (m % kNKB) * 32 * (D * 2)));
            }
        };
        const f32x16 zero = {};
#pragma unroll
        for (int n = 0; n < kLdsLead; ++n) rd(n);
#pragma unroll
        for (int n = 0; n < NP + NQ; ++n) {
            if (n + kLdsLead < NP + NQ) rd(n + kLdsLead);
            if (n < NP) {
                const int t = n / DB, db = n % DB;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[n], pf[t], oacc[db], 0, 0, 0);
            } else {
                const int m = n - NP, ks = m / kNKB, kb = m % kNKB;
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[n], qf[ks], ks == 0 ? zero : s[kb], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Vector phase of tile j: mask, reference update, probabilities. P is
    // first computed against the current reference without the tile's row
    // max: if no lane's share of the row sum exceeds 2^slack, no P exceeds
    // it, so the max could not have exceeded the reference by more than the
    // slack and the reference stays (the result is that of always checking
    // the max). Otherwise, and while a row has no reference yet, the max is
    // taken, the reference moved as needed and P recomputed.
    template <bool WIN>
    __device__ __forceinline__ void vphase(f32x16 (&s)[kNKB], bf16x8 (&pf)[2 * kNKB], int j0, bool masked) {
        __builtin_amdgcn_s_setprio(0);
        if (masked) mask<WIN>(s, j0);
        constexpr float kSumLimit = 256.0f;  // 2^kRescaleSlack
        float ts = 0.0f;
        // (The window instantiation always takes the max: the second
        // probability pass pushed it into spills and measured 5% slower.)
        bool slow = WIN || __builtin_amdgcn_ballot_w64(mref == -INFINITY) != 0;
        if (!slow) {
            ts = probs(s, pf);
            slow = __builtin_amdgcn_ballot_w64(!(ts <= kSumLimit)) != 0;
        }
        if (slow) {
            update_ref(s);
            ts = probs(s, pf);
        }
        lsum += ts;
        // P and the row sum are complete here: keeps the exponentials and
        // sums in this (vector) phase instead of letting the compiler sink
        // them into the next matrix phase, next to their uses.
#pragma unroll
        for (int t = 0; t < 2 * kNKB; ++t) asm volatile("" : : "v"(pf[t]));
        asm volatile("" : : "v"(lsum));
    }
};

// PAGED: queries are the packed rows [cu_q[b], cu_q[b+1]) ([rows, Hq, d]) and
// keys / values the first seq_lens[b] tokens of sequence b in the page pools
// ([pages, Hkv, 16, d]) through the page table; otherwise Q/O are
// [B, Hq, Nq, d] and K/V [B, Hkv, Nk, d]. WINDOW: a sliding window,
// win_left / win_right in FwdParams (contiguous or paged; the window's
// first key tile is a multiple of 128 keys, so page slots stay aligned).
// SPARSE (contiguous mode only): a block mask over 128 x 128 (query, key)
// blocks.
template <int D, bool CAUSAL, bool PAGED, bool WINDOW, bool SPARSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdParams p) {
    static_assert(!SPARSE || kBN == kSparseBlock, "a sparse mask block is one K/V tile");
    constexpr int SB = Stage<D>::kBytesK;  // bytes of one K or V stage
    __shared__ __attribute__((aligned(1024))) char smem_raw[4 * SB + (SPARSE ? kSparseLdsBytes : 0)];
    lds_char* smem = (lds_char*)smem_raw;
    // Stages: K of even tiles, K of odd tiles, V of even tiles, V of odd tiles.
    auto kst = [&](int j) { return smem + (j & 1) * SB; };
    auto vst = [&](int j) { return smem + (2 + (j & 1)) * SB; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int col = lane & 31;

    // ---- workgroup -> (unit, query tile) ----
    int unit, qt;
    {
        const int id = blockIdx.x;
        if (p.xcd_affine) {
            // Workgroups are dealt round-robin to the 8 XCDs; XCD x owns
            // units x, x+8, ...
            const int xcd = id & 7, k = id >> 3;
            const int ux = p.n_units >> 3;  // units per XCD
            if (p.unit_major) {
                // A unit has at least an XCD's worth of query tiles: all of
                // one unit's tiles run together, so the K/V its resident
                // workgroups stream is one unit's, which the XCD's L2 holds.
                const int u = fast_div(k, p.fd_qtiles);
                unit = xcd + 8 * u;
                qt = k - u * p.n_qtiles;
            } else {
                // Few tiles per unit: tile-major over the XCD's units, which
                // (with the heaviest-first order below) balances the rounds.
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
    const int rows_q = kBlockRows * p.qblocks_per_wg;  // queries per tile
    const int qtile0 = qt * rows_q;
    int Nq = p.Nq, Nk = p.Nk;
    size_t qrow0 = 0;  // paged: first packed query row of the sequence
    if constexpr (PAGED) {
        const int c0 = p.cu_q[b];
        Nq = p.cu_q[b + 1] - c0;
        Nk = p.seq_lens[b];
        qrow0 = (size_t)c0;
        if (qtile0 >= Nq) return;  // the grid covers the longest query chunk
    }
    // Row index (into O, and LSE) of query qi of head h.
    auto qrow = [&](int h, int qi) -> size_t {
        if constexpr (PAGED) return (qrow0 + (size_t)qi) * p.Hq + h;
        else return ((size_t)b * p.Hq + h) * Nq + qi;
    };

    // ---- this wave's row block: 32 queries of one head ----
    const int head = g * p.G + hsub * p.heads_per_wg + (wave >> p.qb_log2);
    const int q0 = qtile0 + (wave & (p.qblocks_per_wg - 1)) * kBlockRows;
    // Query i sits at key position i + (Nk - Nq). The right bound (CAUSAL)
    // is that position, or that position + win_right with a WINDOW; the left
    // bound (WINDOW, win_left >= 0) that position - win_left. A workgroup
    // whose first row's left bound is past key 0 starts at the 128-aligned
    // tile holding it: keys are then counted from kofs (the tile loop, copies
    // and masks all use key - kofs).
    const int win_left = WINDOW ? p.win_left : -1;
    int kofs = 0;
    if (WINDOW && win_left >= 0) kofs = max(0, qtile0 + (Nk - Nq) - win_left) / kBN * kBN;
    Nk -= kofs;
    const int shift = Nk - Nq + ((CAUSAL && WINDOW) ? p.win_right : 0);  // right bound: key j <= i + shift

    // Key range of the workgroup and of this wave.
    int wg_kend = Nk, wave_kend = Nk, wave_kmask = Nk;
    if (CAUSAL) {
        const int wg_qlast = min(Nq, qtile0 + rows_q) - 1;
        wg_kend = max(0, min(Nk, wg_qlast + 1 + shift));
        const int wq_last = min(Nq - 1, q0 + kBlockRows - 1);
        wave_kend = max(0, min(Nk, wq_last + 1 + shift));
        wave_kmask = max(0, min(Nk, q0 + 1 + shift));  // keys below this are visible to all rows
    }
    if (q0 >= Nq) wave_kend = 0;  // padding block of a ragged last tile
    const int n_tiles = (wg_kend + kBN - 1) / kBN;
    const int wt = (wave_kend + kBN - 1) / kBN;    // tiles this wave computes (a prefix)
    const int first_masked = wave_kmask / kBN;     // tiles from here on need the mask
    // Window: keys below lo_band lie left of some row's window.
    const int lo_band = win_left >= 0 ? min(q0 + kBlockRows - 1, Nq - 1) + (Nk - Nq) - win_left : 0;

    Wave<D> w;
    {
        const int krow = row_of_mfma_row(col);
        w.koff0 = tile_off<D>(krow, half);
#pragma unroll
        for (int h = 0; h < 2; ++h) w.voff0[h] = tr_off<D>(0, h, lane);
    }
    w.half = half;
    w.lane = lane;
    w.scale_log2 = p.scale_log2;

    // ---- Q fragments (B operand of S^T = K Q^T) ----
    const int qi = q0 + col;
    {
        const uint16_t* qp = p.q + qrow(head, min(qi, Nq - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < Wave<D>::KS; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qi < Nq) x = *reinterpret_cast<const u32x4*>(qp + ks * 16 + half * 8);
            w.qf[ks] = as_bf16x8(x);
        }
    }
    // Causal limit of this lane's query (keys above it are masked).
    w.lim = CAUSAL ? min(Nk - 1, qi + shift) : Nk - 1;
    w.lo = WINDOW && win_left >= 0 ? qi + (Nk - Nq) - win_left : INT32_MIN;
#pragma unroll
    for (int db = 0; db < Wave<D>::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.oacc[db][r] = 0.0f;
    w.mref = -INFINITY;
    w.lsum = 0.0f;

    // K / V row addressing for issue_rows(): contiguous rows of this (batch,
    // K/V head), or pages of the pools at K/V head g with page ids fetched
    // one tile ahead (kpg for the next K copy, vpg for the next V copy).
    constexpr int NI = Stage<D>::kInstPerWave;
    const size_t nk_all = (size_t)(Nk + kofs);  // keys of the (batch, head) in memory
    const uint16_t* kbase = PAGED ? p.k + (size_t)g * 16 * D : p.k + ((size_t)(b * p.Hkv + g) * nk_all + kofs) * D;
    const uint16_t* vbase = PAGED ? p.v + (size_t)g * 16 * D : p.v + ((size_t)(b * p.Hkv + g) * nk_all + kofs) * D;
    const size_t page_stride = (size_t)p.Hkv * 16 * D;
    const int32_t* bt_row = PAGED ? p.bt + (size_t)b * p.maxp + kofs / 16 : nullptr;
    int kpg[NI], vpg[NI];
    // Block-sparse: the workgroup walks a list of the key tiles that any of
    // its row blocks uses, in increasing order. An entry holds the tile index
    // (bits 0-15) and one bit per wave whose row block uses the tile (bits
    // 16-23). Wave w computes list positions [0, wt_w), up to its last own
    // entry (its causal range included); entries in between that are not its
    // own are masked whole. Wave 0 builds the list from the mask bytes.
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    lds_u32* const tlist = (lds_u32*)(smem + 4 * SB);
    int n_steps = n_tiles, w_steps = wt;
    if constexpr (SPARSE) {
        if (wave == 0) {
            const uint8_t* rowp[kWaves];
            int wend[kWaves];
#pragma unroll
            for (int w2 = 0; w2 < kWaves; ++w2) {
                const int h2 = g * p.G + hsub * p.heads_per_wg + (w2 >> p.qb_log2);
                const int q2 = qtile0 + (w2 & (p.qblocks_per_wg - 1)) * kBlockRows;
                int kend = 0;
                if (q2 < Nq) kend = CAUSAL ? max(0, min(Nk, min(Nq - 1, q2 + kBlockRows - 1) + 1 + shift)) : Nk;
                wend[w2] = (kend + kBN - 1) / kBN;
                rowp[w2] = p.bmask + (size_t)b * p.bm_sb + (size_t)h2 * p.bm_sh +
                           (size_t)(min(q2, Nq - 1) / kSparseBlock) * p.n_kb;
            }
            int count = 0;
            int wts[kWaves];
#pragma unroll
            for (int w2 = 0; w2 < kWaves; ++w2) wts[w2] = 0;
            for (int c = 0; c * 64 < n_tiles; ++c) {
                const int t = c * 64 + lane;
                uint32_t flags = 0;
#pragma unroll
                for (int w2 = 0; w2 < kWaves; ++w2)
                    if (t < wend[w2] && rowp[w2][t] != 0) flags |= 1u << w2;
                const uint64_t act = __builtin_amdgcn_ballot_w64(flags != 0);
                const int pos = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
                if (flags != 0) tlist[pos] = (uint32_t)t | (flags << 16);
#pragma unroll
                for (int w2 = 0; w2 < kWaves; ++w2) {
                    const uint64_t bw = __builtin_amdgcn_ballot_w64(((flags >> w2) & 1u) != 0);
                    if (bw != 0) {
                        const int hi = 63 - __builtin_clzll(bw);
                        wts[w2] = count + __builtin_popcountll(act & ((2ull << hi) - 1ull));
                    }
                }
                count += __builtin_popcountll(act);
            }
            if (lane == 0) {
                tlist[kMaxSparseTiles] = (uint32_t)count;
#pragma unroll
                for (int w2 = 0; w2 < kWaves; ++w2) tlist[kMaxSparseTiles + 1 + w2] = (uint32_t)wts[w2];
            }
        }
        __syncthreads();
        n_steps = __builtin_amdgcn_readfirstlane((int)tlist[kMaxSparseTiles]);
        w_steps = __builtin_amdgcn_readfirstlane((int)tlist[kMaxSparseTiles + 1 + wave]);
    }
    auto entry = [&](int t) -> uint32_t { return __builtin_amdgcn_readfirstlane(tlist[t]); };
    // First key of list position / tile t.
    auto tile_key = [&](int t) -> int {
        if constexpr (SPARSE) return (int)(entry(t) & 0xffffu) * kBN;
        else return t * kBN;
    };
    // Tile start this wave masks against (kNoKey: a tile it does not use).
    auto key0 = [&](int t) -> int {
        if constexpr (SPARSE) {
            const uint32_t e = entry(t);
            return ((e >> (16 + wave)) & 1u) ? (int)(e & 0xffffu) * kBN : kNoKey;
        } else {
            return t * kBN;
        }
    };
    auto tile_masked = [&](int t) -> bool {
        if constexpr (SPARSE) {
            const uint32_t e = entry(t);
            return !((e >> (16 + wave)) & 1u) || (int)(e & 0xffffu) >= first_masked;
        } else {
            return t >= first_masked || (WINDOW && t * kBN < lo_band);
        }
    };
    auto issue_k = [&](int t) {
        issue_rows<D>(kbase, PAGED ? kpg : nullptr, page_stride, kst(t), tile_key(t), Nk, wave, lane);
        if (PAGED && t + 1 < n_tiles) page_ids<D>(kpg, bt_row, (t + 1) * kBN, Nk, wave);
    };
    auto issue_v = [&](int t) {
        issue_rows<D>(vbase, PAGED ? vpg : nullptr, page_stride, vst(t), tile_key(t), Nk, wave, lane);
        if (PAGED && t + 1 < n_tiles) page_ids<D>(vpg, bt_row, (t + 1) * kBN, Nk, wave);
    };

    // Ping-pong schedule. Waves w and w+4 share a SIMD; group A = waves 0-3,
    // group B = waves 4-7. Time is cut into slots by workgroup barriers; in
    // each slot one group runs its matrix phase (PV of tile j, then the
    // scores of tile j+1) while the other runs its vector phase (softmax),
    // so each SIMD always has MFMA work from one wave and VALU work from the
    // other:
    //   slot 2j  : A vector phase of tile j   | B matrix phase of tile j-1
    //   slot 2j+1: A matrix phase of tile j   | B vector phase of tile j
    // (B's slot 0 computes the scores of tile 0.) At the start of slot 2j+1
    // the K stage of tile j and the V stage of tile j-1 have no readers left;
    // they receive K of tile j+2 and V of tile j+1, which are first read in
    // slot 2j+3 -- so only the barrier ending an even slot waits for copies.
    if (n_steps > 0) {
        const bool grp_b = wave >= kWaves / 2;
        if constexpr (PAGED) {
            page_ids<D>(kpg, bt_row, 0, Nk, wave);
            page_ids<D>(vpg, bt_row, 0, Nk, wave);
        }
        // At d = 128 with contiguous K/V (not block-sparse) only Q and K of
        // tile 0 are awaited before the first scores; group B copies V of
        // tile 0 and K of tile 1 while group A computes them (both land
        // before the first even barrier, which precedes their first reads).
        constexpr bool kLateFill = !SPARSE && !PAGED && D == 128;
        issue_k(0);
        if constexpr (!kLateFill) {
            issue_v(0);
            if (n_steps > 1) issue_k(1);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        f32x16 s[kNKB];
        bf16x8 pf[2 * kNKB];
        auto end_odd_slot = [&]() {  // LDS reads done; copies may stay in flight
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            asm volatile("s_barrier" ::: "memory");
        };
        // At d = 128 (contiguous or paged K/V, not block-sparse) the copies
        // issued after an even barrier are split unevenly between the groups.
        // Group A goes from them straight into its matrix phase, which is on
        // the tile's critical path; group B goes into its vector phase, which
        // has a few hundred cycles of slack against A's matrix phase. So A's
        // waves copy kCopyA of the 32 1 KiB blocks of the K tile each, and
        // B's waves the other 8 - kCopyA K blocks and 8 V blocks each (even
        // split: 8 each). kCopyA = 4 measured +1.1-1.4% against the even
        // split (3: +1.2%, 5-6: none, 0 and 2: slower). Block i of a tile
        // holds rows 4i..4i+3; a wave's blocks are congruent to it mod 4, so
        // one lane offset (row in the block, swizzled chunk) serves all of
        // them. Full tiles are copied from scalar bases with that one offset,
        // so a copy costs no vector address arithmetic (+1.4% more); a ragged
        // last tile clamps its rows per lane.
        constexpr bool kSkewCopies = !SPARSE && D == 128;
        constexpr int kCopyA = 4;
        const int cp_row = lane / 16;
        const int cp_col = ((lane % 16) ^ swz<D>(4 * (wave & 3) + cp_row)) * 8;
        const uint32_t cp_voff = (uint32_t)(cp_row * D + cp_col) * 2;  // bytes
        auto issue_blocks = [&](const uint16_t* base, lds_char* st, int j0, int first, auto count) {
            constexpr int RPI = 1024 / (D * 2);  // rows per block
            const int uf = __builtin_amdgcn_readfirstlane(first);
            if (j0 + kBN <= Nk) {
#pragma unroll
                for (int m = 0; m < decltype(count)::value; ++m) {
                    const int blk = uf + 4 * m;
                    copy16_to_lds_sbase(cp_voff, base + (size_t)(j0 + blk * RPI) * D, (uint32_t)(uintptr_t)(st + blk * 1024));
                }
            } else {
#pragma unroll
                for (int m = 0; m < decltype(count)::value; ++m) {
                    const int blk = uf + 4 * m;
                    const int key = min(j0 + blk * RPI + cp_row, Nk - 1);
                    copy16_to_lds(base + (size_t)key * D + cp_col, (uint32_t)(uintptr_t)(st + blk * 1024));
                }
            }
        };
        // Paged: group A's K blocks lie in pages 0-3 of a tile, group B's in
        // pages 4-7, and B's V blocks in all 8 (block uw + 4 m holds rows
        // 4 uw + 16 m .. +3: page m, row 4 uw within it). The page ids are
        // read (scalar loads of the table) right before the copies: measured
        // +6.0% over the even split, against +4.9% when V's ids were read one
        // tile ahead and +2.8% when K's were too (more live scalar registers).
        int pidk[4], pidv[8];
        auto issue_blocks_paged = [&](const uint16_t* pool, const int* ids, lds_char* st, int j0, int first, auto count) {
            constexpr int RPI = 1024 / (D * 2);
            const int uf = __builtin_amdgcn_readfirstlane(first);
            if (j0 + kBN <= Nk) {
#pragma unroll
                for (int m = 0; m < decltype(count)::value; ++m) {
                    const int blk = uf + 4 * m;
                    copy16_to_lds_sbase(cp_voff, pool + (size_t)ids[m] * page_stride + (size_t)(4 * (uf & 3)) * D,
                                        (uint32_t)(uintptr_t)(st + blk * 1024));
                }
            } else {
#pragma unroll
                for (int m = 0; m < decltype(count)::value; ++m) {
                    const int blk = uf + 4 * m;
                    const int key = min(j0 + blk * RPI + cp_row, Nk - 1);
                    copy16_to_lds(pool + (size_t)ids[m] * page_stride + (size_t)(key & 15) * D + cp_col,
                                  (uint32_t)(uintptr_t)(st + blk * 1024));
                }
            }
        };
        // copies for slot 2j+1 landed; issue the next ones (group B: is_b)
        auto end_even_slot = [&](int j, auto is_b) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if constexpr (!kSkewCopies) {
                if (j + 2 < n_steps) issue_k(j + 2);
                if (j + 1 < n_steps) issue_v(j + 1);
            } else if constexpr (PAGED) {
                const int uw = wave & 3;
                if constexpr (!decltype(is_b)::value) {
                    if (j + 2 < n_steps) {
                        page_ids_run(pidk, bt_row, (j + 2) * kBN, 0, Nk);
                        issue_blocks_paged(kbase, pidk, kst(j + 2), (j + 2) * kBN, uw, std::integral_constant<int, kCopyA>{});
                    }
                } else {
                    if (j + 2 < n_steps) {
                        page_ids_run(pidk, bt_row, (j + 2) * kBN, kCopyA, Nk);
                        issue_blocks_paged(kbase, pidk, kst(j + 2), (j + 2) * kBN, 4 * kCopyA + uw,
                                           std::integral_constant<int, 8 - kCopyA>{});
                    }
                    if (j + 1 < n_steps) {
                        page_ids_run(pidv, bt_row, (j + 1) * kBN, 0, Nk);
                        issue_blocks_paged(vbase, pidv, vst(j + 1), (j + 1) * kBN, uw, std::integral_constant<int, 8>{});
                    }
                }
            } else {
                // (tile t starts at key t * kBN: no sparse tile list here)
                const int uw = wave & 3;
                if constexpr (!decltype(is_b)::value) {
                    if (j + 2 < n_steps)
                        issue_blocks(kbase, kst(j + 2), (j + 2) * kBN, uw, std::integral_constant<int, kCopyA>{});
                } else {
                    if (j + 2 < n_steps)
                        issue_blocks(kbase, kst(j + 2), (j + 2) * kBN, 4 * kCopyA + uw,
                                     std::integral_constant<int, 8 - kCopyA>{});
                    if (j + 1 < n_steps) issue_blocks(vbase, vst(j + 1), (j + 1) * kBN, uw, std::integral_constant<int, 8>{});
                }
            }
        };
        // No MFMA block is conditional inside a loop (a conditional MFMA
        // update makes the compiler copy the accumulators every iteration):
        // each group runs the slots of its own tiles [0, w_steps) -- the last one
        // peeled -- and then only takes part in the remaining barriers.
        int j = 0;
        if (!grp_b) {
            if (w_steps > 0) w.qk(s, kst(0));
            for (; j + 1 < w_steps; ++j) {
                if (j > 0) end_odd_slot();
                w.template vphase<WINDOW>(s, pf, key0(j), tile_masked(j));
                end_even_slot(j, std::false_type{});
                w.pv_qk(pf, vst(j), s, kst(j + 1));
            }
            if (j < w_steps) {
                if (j > 0) end_odd_slot();
                w.template vphase<WINDOW>(s, pf, key0(j), tile_masked(j));
                end_even_slot(j, std::false_type{});
                w.pv_tile(pf, vst(j));
                ++j;
            }
            for (;; ++j) {
                if (j > 0) end_odd_slot();
                if (j == n_steps) break;
                end_even_slot(j, std::false_type{});
            }
        } else {
            if constexpr (kLateFill) {
                issue_blocks(vbase, vst(0), 0, wave & 3, std::integral_constant<int, 8>{});
                if (n_steps > 1) issue_blocks(kbase, kst(1), kBN, wave & 3, std::integral_constant<int, 8>{});
            }
            if (w_steps > 0) w.qk(s, kst(0));
            end_even_slot(0, std::true_type{});
            if (w_steps > 0) w.template vphase<WINDOW>(s, pf, key0(0), tile_masked(0));
            for (j = 1; j < w_steps; ++j) {
                end_odd_slot();
                w.pv_qk(pf, vst(j - 1), s, kst(j));
                end_even_slot(j, std::true_type{});
                w.template vphase<WINDOW>(s, pf, key0(j), tile_masked(j));
            }
            bool done = false;
            if (w_steps > 0) {  // j == w_steps: the last PV
                end_odd_slot();
                w.pv_tile(pf, vst(j - 1));
                if (j == n_steps) done = true;
                else end_even_slot(j++, std::true_type{});
            }
            if (!done)
                for (;; ++j) {
                    end_odd_slot();
                    if (j == n_steps) break;
                    end_even_slot(j, std::true_type{});
                }
        }
    }

    __builtin_amdgcn_s_setprio(0);

    // ---- epilogue: O = O^T / l (transposed back on store), LSE = ln 2 * m + ln l ----
    const float l = w.lsum + other_half(w.lsum);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    // The lane, its query and its row are recomputed here from the lane id
    // (opaque to the compiler), so none of the prologue's values has to stay
    // live (and spill) across the loop.
    int el = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(el));
    const int ehalf = el >> 5, eqi = q0 + (el & 31);
    if (eqi < Nq) {
        const int half = ehalf, qi = eqi;
        const size_t row = qrow(head, qi);
        uint16_t* op = p.o + row * D;
#pragma unroll
        for (int db = 0; db < Wave<D>::DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dim = db * 32 + r4 * 8 + half * 4;
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(w.oacc[db][r4 * 4 + e] * inv);
                *reinterpret_cast<bf16x4*>(op + dim) = ov;
            }
        if (half == 0) p.lse[row] = l > 0.0f ? (w.mref * kLn2 + logf(l)) : -INFINITY;
    }
}

int pow2_divisor_upto8(int G) {
    int h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

template <int D, bool CAUSAL, bool PAGED, bool WINDOW, bool SPARSE>
hipError_t launch_t(const FwdParams& p, int grid, hipStream_t stream) {
    if (trace_on())
        trace("fa_fwd_kernel<d=%d, causal=%d, paged=%d, window=%d, sparse=%d> grid=%d block=%d "
              "(units=%d x query tiles=%d, heads per workgroup=%d, xcd_affine=%d, unit_major=%d)",
              D, (int)CAUSAL, (int)PAGED, (int)WINDOW, (int)SPARSE, grid, kThreads, p.n_units, p.n_qtiles,
              p.heads_per_wg, p.xcd_affine, p.unit_major);
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, PAGED, WINDOW, SPARSE>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool PAGED, bool WINDOW, bool SPARSE>
hipError_t launch_d(const FwdParams& p, int grid, hipStream_t stream) {
    return p.causal ? launch_t<D, true, PAGED, WINDOW, SPARSE>(p, grid, stream)
                    : launch_t<D, false, PAGED, WINDOW, SPARSE>(p, grid, stream);
}

template <bool PAGED, bool WINDOW, bool SPARSE>
hipError_t launch_any(const FwdParams& p, int d, int grid, hipStream_t stream) {
    return d == 128 ? launch_d<128, PAGED, WINDOW, SPARSE>(p, grid, stream)
                    : launch_d<64, PAGED, WINDOW, SPARSE>(p, grid, stream);
}

// Group packing and grid size (shared by both modes); Nq is the longest query
// chunk in paged mode.
void plan(FwdParams& p, int B, int Hq, int Hkv, int Nq) {
    p.G = Hq / Hkv;
    p.heads_per_wg = pow2_divisor_upto8(p.G);
    p.qblocks_per_wg = kBlocksPerWG / p.heads_per_wg;
    p.n_hsub = p.G / p.heads_per_wg;
    const int rows_q = kBlockRows * p.qblocks_per_wg;
    p.n_qtiles = (Nq + rows_q - 1) / rows_q;
    p.n_units = B * Hkv * p.n_hsub;
    p.xcd_affine = (p.n_units % 8 == 0) ? 1 : 0;
    p.unit_major = (p.n_qtiles >= kCusPerXcd) ? 1 : 0;
    p.qb_log2 = 0;
    while ((1 << p.qb_log2) < p.qblocks_per_wg) ++p.qb_log2;
    p.fd_qtiles = make_fastdiv(p.n_qtiles);
    p.fd_ux = make_fastdiv(p.n_units >= 8 ? p.n_units >> 3 : 1);
    p.fd_units = make_fastdiv(p.n_units);
    p.fd_hsub = make_fastdiv(p.n_hsub);
    p.fd_hkv = make_fastdiv(Hkv);
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
    FwdParams p = {};
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
    plan(p, a.B, a.Hq, a.Hkv, a.Nq);
    // A window runs the WINDOW kernels; a right bound (causal, or a right
    // window) their CAUSAL instantiation.
    const bool window = a.window_left >= 0 || (!a.causal && a.window_right >= 0);
    p.causal = (a.causal || a.window_right >= 0) ? 1 : 0;
    p.win_right = a.causal ? 0 : a.window_right;
    p.win_left = a.window_left;
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    const long long grid = (long long)p.n_units * p.n_qtiles;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.block_mask != nullptr) {  // block-sparse (no window)
        p.bmask = a.block_mask;
        p.bm_sb = a.mask_stride_b;
        p.bm_sh = a.mask_stride_h;
        p.n_kb = (a.Nk + kSparseBlock - 1) / kSparseBlock;
        if (window || p.n_kb > kMaxSparseTiles) return hipErrorInvalidValue;
        return launch_any<false, false, true>(p, a.d, (int)grid, stream);
    }
    return window ? launch_any<false, true, false>(p, a.d, (int)grid, stream)
                  : launch_any<false, false, false>(p, a.d, (int)grid, stream);
}

hipError_t launch_paged_prefill(const PagedPrefillArgs& a, hipStream_t stream) {
    FwdParams p = {};
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k_pool);
    p.v = static_cast<const uint16_t*>(a.v_pool);
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.max_q_len; p.Nk = 0;
    p.bt = a.block_table;
    p.seq_lens = a.seq_lens;
    p.cu_q = a.cu_seqlens_q;
    p.maxp = a.max_pages_per_seq;
    plan(p, a.B, a.Hq, a.Hkv, a.max_q_len);
    // A window runs the PAGED + WINDOW kernels (as for launch_forward).
    const bool window = a.window_left >= 0 || (!a.causal && a.window_right >= 0);
    p.causal = (a.causal || a.window_right >= 0) ? 1 : 0;
    p.win_right = a.causal ? 0 : a.window_right;
    p.win_left = a.window_left;
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    const long long grid = (long long)p.n_units * p.n_qtiles;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    return window ? launch_any<true, true, false>(p, a.d, (int)grid, stream)
                  : launch_any<true, false, false>(p, a.d, (int)grid, stream);
}

}  // namespace fa
