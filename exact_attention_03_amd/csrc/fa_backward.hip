// Attention backward for gfx950 (CDNA4): dQ, dK, dV of
// O = softmax(scale * Q K^T + mask) V for an incoming gradient dO.
//
// Method (page "Flash Attention : pourquoi ton GPU utilise 85% de VRAM",
// section "Ce que fait Flash Attention": the backward recomputes the
// attention matrix block by block instead of storing it). With the row
// log-sum-exp L saved by the forward, P = exp(scale * Q K^T - L) is
// recomputed tile by tile in registers; with Dr = rowsum(dO * O), which
// equals rowsum(dP * P) because O = P V,
//     dS = P * (dO V^T - Dr),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Nothing of size Nq x Nk is ever written to memory.
//
// Three kernels, all on v_mfma_f32_32x32x16_bf16 with bf16 operands (P and
// dS rounded to bf16, as the forward rounds P) and fp32 accumulation:
//   * fa_bwd_pre: Dr per query row, and the LSE in exp2 units, into the
//     caller's workspace (HBM-bound, one pass over dO and O).
//   * fa_bwd_dq: the forward's structure. A workgroup is 8 row blocks of 32
//     queries sharing one K/V head; each lane holds one query. Per 64-key
//     tile: S^T = K Q^T and dP^T = V dO^T (Q and dO fragments stay in
//     registers; K and V rows are read in the permuted order that makes each
//     lane's results the B operand of the next product), P^T and dS^T
//     elementwise, then dQ^T += K^T dS^T with K^T from the transposing LDS
//     read. As in the forward, the two wave groups ping-pong across barrier
//     slots (one group's MFMAs against the other's elementwise work); K has
//     a four-stage LDS ring, V two stages.
//   * fa_bwd_dkdv: the mirror image. A workgroup owns 128 keys of one K/V
//     head (K and V staged in LDS once); wave w holds keys 32*(w%4) ..+31,
//     one per lane, and the query half w/4 of every 64-query tile. It walks
//     the query tiles (last first) of all G query heads of the K/V head (so
//     GQA needs no atomics), computing S = Q K^T and dP = dO V^T with Q / dO
//     rows read in the permuted order, then dV^T += dO^T P and dK^T += Q^T dS
//     with the transposing reads of the staged Q / dO tile. A step's Q / dO
//     rows and its LSE / Dr values arrive by LDS DMA one step ahead. The two
//     query halves are summed through LDS at the end.
// Masked elements get a -inf exponent (a select, no control flow).
// Deterministic: no atomics anywhere.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "fa_kernels.h"
#include "fa_divide.h"
#include "fa_lds.h"

namespace fa {
namespace {

using namespace lds;

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kRows = 32;     // queries (dq) or keys (dkdv) per wave
constexpr int kKT = 64;       // keys per K/V tile of the dq kernel
constexpr int kQT = 64;       // queries per Q/dO tile of the dkdv kernel
constexpr int kKW = 128;      // keys per dkdv workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLead = 2;      // operand pairs read ahead of their MFMAs
constexpr int kNoBound = 1 << 29;  // a window side without a bound (keeps index sums in int range)

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* dr;    // rowsum(dO * O), [B, Hq, Nq] (workspace)
    float* lse2;  // LSE in exp2 units, lse2_of(lse), [B, Hq, Nq] (workspace, after dr)
    int B, Hq, Hkv, Nq, Nk, G;
    int heads_per_wg, qblocks_per_wg, n_hsub, n_qtiles, n_units;  // dq grid (as the forward's)
    int n_ktiles;                                                // dkdv grid: keys / kKW
    int qb_log2;                                                 // log2(qblocks_per_wg)
    // Divisions of the grid mappings and of the dK/dV steps: by the dq
    // grid's n_units, n_hsub, Hkv, the dK/dV grid's B * Hkv, G and nseg.
    FastDiv fd_units, fd_hsub, fd_hkv, fd_kvunits, fd_G, fd_nseg;
    // Sliding window (WINDOW kernels): query i at key position p = i + Nk - Nq
    // sees keys [p - win_left, p + win_right]; a negative bound is none.
    int win_left, win_right;
    float scale, scale_log2;
    // Block mask (SPARSE kernels): entry (b, h, qb, kb) at
    // bmask[b * bm_sb + h * bm_sh + qb * n_kb + kb], over blocks of
    // kSparseMaskBlock queries and keys; nonzero = the block pair attends.
    const uint8_t* bmask;
    long long bm_sb, bm_sh;
    int n_kb;
    // SPARSE dK/dV runs: the visible steps of one key block are cut into at
    // most nseg runs; a key block with more than one run leaves one fp32
    // partial per run (partial, 2 * kKW * d floats per slot: dK then dV,
    // unscaled), a flag per run saying whether it had a visible step
    // (seg_flags) and its number of runs (seg_count), all summed by
    // fa_bwd_dkdv_combine. Slots [B * Hkv][key blocks][nseg]; the partials,
    // flags and counts exist only for nseg > 1.
    int nseg;
    float* partial;
    uint32_t* seg_flags;
    uint32_t* seg_count;
};

static_assert(kSparseMaskBlock == 2 * kKT && kSparseMaskBlock == 2 * kQT && kSparseMaskBlock == kKW,
              "a mask block is two dq key tiles, two dkdv query tiles and one dkdv workgroup");
// Mask entry of query block qb and key block kb for query head h of batch b.
__device__ __forceinline__ const uint8_t* mask_row(const BwdParams& p, int b, int h, int qb) {
    return p.bmask + (size_t)b * p.bm_sb + (size_t)h * p.bm_sh + (size_t)qb * p.n_kb;
}
typedef __attribute__((address_space(3))) uint64_t lds_u64;
// A 64-bit ballot as one uniform value.
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// LSE in exp2 units for P = exp2(s * scale_log2 - lse2); +inf for a row
// with no visible key (its P is then 0 everywhere, never inf - inf).
__device__ __forceinline__ float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ---- Dr = rowsum(dO * O), and the LSE in exp2 units ------------------------
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre(BwdParams p, long long rows) {
    constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
    const long long row = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int sub = threadIdx.x % LPR;
    float acc = 0.0f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + row * D + sub * 8);
        const u32x4 b = *reinterpret_cast<const u32x4*>(p.o + row * D + sub * 8);
        const bf16x8 x = as_bf16x8(a), y = as_bf16x8(b);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && sub == 0) {
        p.dr[row] = acc;
        p.lse2[row] = lse2_of(p.lse[row]);
    }
}

// ---- dQ ----------------------------------------------------------------------
// WINDOW: the sliding window's bounds (p.win_left, p.win_right) replace the
// causal mask (the host folds causal into win_right = 0).
// SPARSE: the block mask. Each wave's 32 queries lie in one mask query block
// and each 64-key tile in one key block, so a wave sees a tile whole or not
// at all. The workgroup visits only the tiles of key blocks that some wave
// sees (both tiles of such a block); a wave that does not see a visited
// tile masks it whole.
template <int D, bool CAUSAL, bool WINDOW, bool SPARSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq(BwdParams p) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int SB = kKT * D * 2;  // bytes of one K or V stage
    // K stages: tile j is read until two slots after its scores (by the
    // products dQ^T += K^T dS^T), so the ring needs three; it has four, as a
    // stage index of j % 3 made the compiler keep per-stage address vectors
    // (and spill) where j & 3 costs nothing. Two V stages.
    // SPARSE: after the stages, one bitmap per wave of the key blocks it
    // sees (bit kb of word kb / 64).
    constexpr int kMapWords = kSparseMaxKeyBlocks / 64;
    __shared__ __attribute__((aligned(1024))) char smem_raw[6 * SB + (SPARSE ? kWaves * kMapWords * 8 : 0)];
    lds_char* smem = (lds_char*)smem_raw;
    // Ring positions: K stage r & 3, V stage r & 1.
    auto kst = [&](int r) { return smem + (r & 3) * SB; };
    auto vst = [&](int r) { return smem + (4 + (r & 1)) * SB; };
    lds_u64* const kmap = (lds_u64*)(smem + 6 * SB);

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int id = blockIdx.x;
    int qt = fast_div(id, p.fd_units);
    const int unit = id - qt * p.n_units;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest first
    // unit = hsub + n_hsub * (g + Hkv * b)
    const int uh = fast_div(unit, p.fd_hsub);
    const int hsub = unit - uh * p.n_hsub;
    const int b = fast_div(uh, p.fd_hkv);
    const int g = uh - b * p.Hkv;
    const int rows_q = kRows * p.qblocks_per_wg;
    const int qtile0 = qt * rows_q;
    const int head = g * p.G + hsub * p.heads_per_wg + (wave >> p.qb_log2);
    const int q0 = qtile0 + (wave & (p.qblocks_per_wg - 1)) * kRows;
    const int Nq = p.Nq, Nk = p.Nk, shift = Nk - Nq;
    // Visible keys of query i: [i + shift - left, i + shift + right].
    const int right = WINDOW ? (p.win_right >= 0 ? p.win_right : kNoBound) : (CAUSAL ? 0 : kNoBound);
    const int left = WINDOW && p.win_left >= 0 ? p.win_left : kNoBound;
    int kend = Nk;  // keys the workgroup needs: [kbeg, kend)
    if (CAUSAL || WINDOW) kend = max(0, min(Nk, min(Nq, qtile0 + rows_q) + shift + right));
    const int kbeg = WINDOW ? min(kend, max(0, qtile0 + shift - left)) : 0;
    const int t0 = kbeg / kKT;  // first key tile
    const int nt = (kend + kKT - 1) / kKT;

    // This lane's query: Q^T and dO^T fragments (B operands), LSE, Dr.
    const int qi = q0 + col;
    const size_t row = ((size_t)b * p.Hq + head) * Nq + min(qi, Nq - 1);
    bf16x8 qf[KS], dof[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(p.q + row * D + ks * 16 + half * 8));
        dof[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(p.dout + row * D + ks * 16 + half * 8));
    }
    const float lse2 = qi < Nq ? p.lse2[row] : INFINITY;
    const float dr = qi < Nq ? p.dr[row] : 0.0f;
    const int lim = min(Nk - 1, qi + shift + right);  // last visible key
    const int lo = WINDOW ? qi + shift - left : 0;      // first visible key

    // Operand offsets: K / V rows in MFMA-row order (A operand), K^T reads.
    int roff[KS], troff[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = tile_off<D>(row_of_mfma_row(col), 2 * ks + half);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) troff[db][h] = tr_off<D>(db, h, lane);

    const uint16_t* kb = p.k + ((size_t)b * p.Hkv + g) * Nk * D;
    const uint16_t* vb = p.v + ((size_t)b * p.Hkv + g) * Nk * D;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

    // Per tile j: the matrix work S^T, dP^T (scores), the elementwise work
    // dS^T, and the products dQ^T += K^T dS^T.
    f32x16 s[kKT / 32], dp[kKT / 32];
    bf16x8 dsb[kKT / 16];
    // S^T and dP^T of the tile at ring position r: product n uses the K and V
    // rows of 32-key block n / KS at k-step n % KS, read kLead products ahead.
    auto scores = [&](int r) {
        typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
        const lds_char* ks_ = kst(r);
        const lds_char* vs_ = vst(r);
        constexpr int NP = (kKT / 32) * KS;
        bf16x8 kf[NP], vf[NP];
        auto rd = [&](int n) {
            const int o = roff[n % KS] + (n / KS) * 32 * D * 2;
            kf[n] = *reinterpret_cast<const lds_bf16x8*>(ks_ + o);
            vf[n] = *reinterpret_cast<const lds_bf16x8*>(vs_ + o);
        };
        const f32x16 zero = {};
#pragma unroll
        for (int n = 0; n < kLead && n < NP; ++n) rd(n);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            if (n + kLead < NP) rd(n + kLead);
            const int kb2 = n / KS, ks = n % KS;
            s[kb2] = mfma32(kf[n], qf[ks], ks == 0 ? zero : s[kb2]);
            dp[kb2] = mfma32(vf[n], dof[ks], ks == 0 ? zero : dp[kb2]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // dS^T = P^T (dP^T - Dr) of tile j; register r of block kb2 holds key
    // 32*kb2 + 16*(r/8) + 8*half + r%8 of the tile. Masked keys get a -inf
    // exponent (a select, no per-element control flow).
    auto elementwise = [&](int j) {
        __builtin_amdgcn_s_setprio(0);
        int hi = lim;  // last key of the tile this lane's query may see
        if constexpr (SPARSE) {
            const int kbk = j >> 1;
            if (!((uniform64(kmap[wave * kMapWords + (kbk >> 6)]) >> (kbk & 63)) & 1u)) hi = -1;
        }
#pragma unroll
        for (int kb2 = 0; kb2 < kKT / 32; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j * kKT + kb2 * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
                float x = __builtin_fmaf(s[kb2][r], p.scale_log2, -lse2);
                x = (key <= hi && (!WINDOW || key >= lo)) ? x : -INFINITY;
                const float pr = __builtin_amdgcn_exp2f(x);
                dsb[kb2 * 2 + (r >> 3)][r & 7] = (__bf16)(pr * (dp[kb2][r] - dr));
            }
        // dS is complete here: keeps the work in this phase instead of letting
        // the compiler sink it into the next matrix phase.
#pragma unroll
        for (int t = 0; t < kKT / 16; ++t) asm volatile("" : : "v"(dsb[t]));
    };
    // dQ^T += K^T dS^T over the four 16-key slices of the tile at ring
    // position r (K^T read kLead products ahead). Raises the wave's priority
    // for its matrix phase.
    auto products = [&](int r) {
        __builtin_amdgcn_s_setprio(1);
        const lds_char* ks_ = kst(r);
        constexpr int NP = (kKT / 16) * DB;
        bf16x8 kt[NP];
#pragma unroll
        for (int n = 0; n < kLead; ++n) kt[n] = read_tr<D>(ks_, troff, n % DB, n / DB);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            if (n + kLead < NP) kt[n + kLead] = read_tr<D>(ks_, troff, (n + kLead) % DB, (n + kLead) / DB);
            acc[n % DB] = mfma32(kt[n], dsb[n / DB], acc[n % DB]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Ping-pong (the forward's schedule). Group A = waves 0-3, group B =
    // waves 4-7, one of each per SIMD. Workgroup barriers cut time into
    // slots; in each slot one group runs its matrix phase (products of tile
    // j-1, then the scores of tile j) while the other runs its elementwise
    // phase, so the matrix cores are not idle during the exponentials:
    //   slot 2j  : A elementwise of tile j  | B products j-1, scores j
    //   slot 2j+1: A products j, scores j+1 | B elementwise of tile j
    // (slot 0: both groups compute the scores of tile 0). K of tile j is read
    // until slot 2j+2, V of tile j until slot 2j. At the start of slot 2j+1
    // the stages of K(j-2) and V(j) are free and receive K(j+2) and V(j+2),
    // first read in slot 2j+3: only the barrier ending an even slot waits for
    // copies. Both groups pass the same 2*nt barriers, even and odd in turn.
    // (Here j counts visited tiles: the ring position. SPARSE visits a
    // subsequence of the tiles, in increasing order.)
    auto end_odd_slot = [&]() {  // LDS reads done; copies may stay in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
    };
    // Group A issues the copies: its even-slot barrier falls between its
    // elementwise work and its products, where few registers are live
    // (group B's falls right after its scores).
    // A full tile is copied from scalar bases with the wave's one lane
    // offset; the ragged last one with per-lane clamped rows (from an
    // opaque lane index, so none of its address arithmetic is hoisted
    // into registers held across the loop).
    const uint32_t cpoff = stage_lane_offset<D, kWaves / 2>(wave, lane);
    auto end_even_slot = [&](int r2, int j2) {  // tile j2 (ring position r2) copied after this
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave < kWaves / 2 && j2 < nt) {
            if ((j2 + 1) * kKT <= Nk) {
                stage_rows_full<D, kKT, kWaves / 2>(kb, kst(r2), j2 * kKT, cpoff, wave);
                stage_rows_full<D, kKT, kWaves / 2>(vb, vst(r2), j2 * kKT, cpoff, wave);
            } else {
                int l = lane;
                asm volatile("" : "+v"(l));
                stage_rows<D, kKT, kWaves / 2>(kb, kst(r2), j2 * kKT, Nk, wave, l);
                stage_rows<D, kKT, kWaves / 2>(vb, vst(r2), j2 * kKT, Nk, wave, l);
            }
        }
    };
    if constexpr (!SPARSE) {
        if (nt > t0) {
            stage_rows<D, kKT, kWaves>(kb, kst(t0), t0 * kKT, Nk, wave, lane);
            stage_rows<D, kKT, kWaves>(vb, vst(t0), t0 * kKT, Nk, wave, lane);
            if (t0 + 1 < nt) {
                stage_rows<D, kKT, kWaves>(kb, kst(t0 + 1), (t0 + 1) * kKT, Nk, wave, lane);
                stage_rows<D, kKT, kWaves>(vb, vst(t0 + 1), (t0 + 1) * kKT, Nk, wave, lane);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // Each group's loop body is scores(j), elementwise(j), products(j)
            // with the barriers placed for its offset, so only the accumulators
            // and the fragments of Q and dO live across iterations.
            if (wave < kWaves / 2) {
                for (int j = t0; j < nt; ++j) {
                    scores(j);            // slot 2j-1 (slot 0 for the first tile)
                    if (j > t0) end_odd_slot();
                    elementwise(j);       // slot 2j
                    end_even_slot(j + 2, j + 2);
                    products(j);          // slot 2j+1
                }
                end_odd_slot();
            } else {
                for (int j = t0; j < nt; ++j) {
                    scores(j);            // slot 2j
                    end_even_slot(j + 2, j + 2);
                    elementwise(j);       // slot 2j+1
                    end_odd_slot();
                    products(j);          // slot 2j+2
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    } else {
        // Each wave's bitmap of the key blocks below kend its mask row sets.
        const int kb_end = (kend + kSparseMaskBlock - 1) / kSparseMaskBlock;
        const uint8_t* mrow = mask_row(p, b, head, min(q0, Nq - 1) / kSparseMaskBlock);
        for (int c = 0; c * 64 < kb_end; ++c) {
            const int kbk = c * 64 + lane;
            const uint64_t bits = __builtin_amdgcn_ballot_w64(q0 < Nq && kbk < kb_end && mrow[kbk] != 0);
            if (lane == 0) kmap[wave * kMapWords + c] = bits;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // The first key block >= kbk that some wave sees (kb_end: none), and
        // the visited tile after tile j (nt: none): the second tile of j's
        // block, else the first tile of the next seen block.
        auto next_block = [&](int kbk) -> int {
            for (int c = kbk >> 6; c * 64 < kb_end; ++c) {
                uint64_t u = 0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) u |= kmap[w * kMapWords + c];
                u = uniform64(u);
                if (c == (kbk >> 6)) u &= ~0ull << (kbk & 63);
                if (u != 0) return c * 64 + __builtin_ctzll(u);
            }
            return kb_end;
        };
        auto next_tile = [&](int j) -> int {
            if (!(j & 1) && j + 1 < nt) return j + 1;
            const int kbk = next_block((j >> 1) + 1);
            return kbk < kb_end ? 2 * kbk : nt;
        };
        const int kb0 = next_block(0);
        int j = kb0 < kb_end ? 2 * kb0 : nt;
        if (j < nt) {
            int j1 = next_tile(j), j2 = next_tile(j1);  // the next two visited tiles
            stage_rows<D, kKT, kWaves>(kb, kst(0), j * kKT, Nk, wave, lane);
            stage_rows<D, kKT, kWaves>(vb, vst(0), j * kKT, Nk, wave, lane);
            if (j1 < nt) {
                stage_rows<D, kKT, kWaves>(kb, kst(1), j1 * kKT, Nk, wave, lane);
                stage_rows<D, kKT, kWaves>(vb, vst(1), j1 * kKT, Nk, wave, lane);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (wave < kWaves / 2) {
                for (int r = 0; j < nt; ++r) {
                    scores(r);
                    if (r > 0) end_odd_slot();
                    elementwise(j);
                    end_even_slot(r + 2, j2);
                    products(r);
                    j = j1; j1 = j2; j2 = next_tile(j2);
                }
                end_odd_slot();
            } else {
                for (int r = 0; j < nt; ++r) {
                    scores(r);
                    end_even_slot(r + 2, j2);
                    elementwise(j);
                    end_odd_slot();
                    products(r);
                    j = j1; j1 = j2; j2 = next_tile(j2);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    }

    // dQ = scale * (dQ^T)^T, one query row per lane.
    if (qi < Nq) {
        uint16_t* op = p.dq + row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[db][r4 * 4 + e] * p.scale);
                *reinterpret_cast<bf16x4*>(op + db * 32 + r4 * 8 + half * 4) = ov;
            }
    }
}

// ---- dK, dV ------------------------------------------------------------------
template <int D>
struct DkdvLds {
    static constexpr int kKV = kKW * D * 2;   // K (or V) rows of the workgroup
    static constexpr int kQ = kQT * D * 2;    // one Q (or dO) stage
    static constexpr int kRowVals = kQT * 4;  // one stage of lse2 (or Dr) values
    static constexpr int kBytes = 2 * kKV + 4 * kQ + 4 * kRowVals;
    static constexpr int kReduce = (kWaves / 2) * 2 * (D / 32) * 16 * 64 * 4;  // final pair sums
    static constexpr int kTotal = kBytes > kReduce ? kBytes : kReduce;
};

// SPARSE: the block mask. The workgroup's 128 keys are one mask key block
// and a step's 64 queries lie in one query block, so a step is visible whole
// or not at all; the workgroup walks only the visible steps, from a bitmap
// of all the key block's steps. A key block with more than kSparseRun
// visible steps is shared by up to p.nseg workgroups, each taking an equal
// run of them and leaving an fp32 partial for fa_bwd_dkdv_combine: a key
// block that every query block sees (a global column) does not outlast the
// rest of the grid. (Measured on the causal GQA 64/8 N=8192 shape: runs of
// at most 128 steps balanced local, local + global and random masks better
// than 256 or 512.)
constexpr int kSparseRun = 128;          // visible steps per run, when p.nseg allows
constexpr int kSparseMaxSteps = 131072;  // most steps (G * query tiles) per key block
static_assert(kSparseMaxSteps == kSparseMaxBackwardSteps, "the bitmap holds every step of a key block");

template <int D, bool CAUSAL, bool WINDOW, bool SPARSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv(BwdParams p) {
    using L = DkdvLds<D>;
    constexpr int KS = D / 16, DB = D / 32;
    __shared__ __attribute__((aligned(1024))) char smem_raw[L::kTotal + (SPARSE ? kSparseMaxSteps / 8 : 0)];
    lds_char* smem = (lds_char*)smem_raw;
    lds_char* kt_ = smem;
    lds_char* vt_ = smem + L::kKV;
    // Stages of ring position r (r & 1).
    auto qst = [&](int r) { return smem + 2 * L::kKV + (r & 1) * L::kQ; };
    auto dost = [&](int r) { return smem + 2 * L::kKV + (2 + (r & 1)) * L::kQ; };
    typedef __attribute__((address_space(3))) float lds_float;
    // Row values of ring position r, query half h: the half's 32 LSE (exp2
    // units), then its 32 Dr values.
    auto rvst = [&](int r, int h) {
        return (lds_float*)(smem + 2 * L::kKV + 4 * L::kQ + ((r & 1) * 2 + h) * L::kRowVals);
    };

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb4 = wave & 3;   // this wave's 32-key block
    const int qh = wave >> 2;   // this wave's query half of each tile

    const int id = blockIdx.x;
    const int n_units = p.B * p.Hkv;
    const int id_hi = fast_div(id, p.fd_kvunits);
    const int unit = id - id_hi * n_units;
    // SPARSE: a key block's nseg workgroups are adjacent (the first key
    // blocks, the heaviest under a causal mask, first), its runs dealt to
    // them in an order rotated per key block. Workgroups past a key block's
    // runs end at once; with them always in the same place of each group
    // (every second workgroup, for two runs) the kernel took up to twice as
    // long (measured), as if the workgroups an XCD deals to some of its
    // shader engines were only those.
    const int kt = SPARSE ? fast_div(id_hi, p.fd_nseg) : id_hi;  // heaviest (earliest keys) first under the causal mask
    const int seg = SPARSE ? (int)(((unsigned)(id_hi - kt * p.nseg) + (((unsigned)kt * 2654435761u) >> 16)) %
                                   (unsigned)p.nseg)
                           : 0;
    const int b = fast_div(unit, p.fd_hkv), g = unit - b * p.Hkv;
    const int k0 = kt * kKW;
    const int Nq = p.Nq, Nk = p.Nk, shift = Nk - Nq;
    const int n_qt = (Nq + kQT - 1) / kQT;
    // Key j is visible to the queries [j - shift - right, j - shift + left].
    const int right = WINDOW ? (p.win_right >= 0 ? p.win_right : kNoBound) : (CAUSAL ? 0 : kNoBound);
    const int left = WINDOW && p.win_left >= 0 ? p.win_left : kNoBound;
    const int t_lo = (CAUSAL || WINDOW) ? min(n_qt, max(0, k0 - shift - right) / kQT) : 0;
    int t_hi = n_qt - 1;  // query tiles [t_lo, t_hi]
    if (WINDOW && left < kNoBound) {
        const int qmax = k0 + kKW - 1 - shift + left;  // last query any key of the workgroup sees
        t_hi = qmax < 0 ? -1 : min(n_qt - 1, qmax / kQT);
    }
    const int n_it = p.G * max(0, t_hi - t_lo + 1);  // (query tile, head) steps

    const uint16_t* kbase = p.k + ((size_t)b * p.Hkv + g) * Nk * D;
    const uint16_t* vbase = p.v + ((size_t)b * p.Hkv + g) * Nk * D;
    // Step `it`: query tile t_hi - it / G of head g*G + it % G. Every
    // workgroup walks the tiles from the last one down (to its own first),
    // all G heads of a tile together, so the workgroups an XCD runs at once
    // read the same Q / dO tiles at about the same time and share them in L2.
    auto step_rows = [&](int it, size_t& rowbase, int& t) {
        const int tq = fast_div(it, p.fd_G);
        const int hh = it - tq * p.G;
        t = t_hi - tq;
        rowbase = ((size_t)b * p.Hq + g * p.G + hh) * Nq;
    };
    // Copies of query half h (rows 32h .. 32h+31) of step it into ring
    // position r, issued by the four waves of group h: the half's Q and dO
    // rows, and its 32 LSE (exp2 units) and 32 Dr values (one wave, 4 bytes
    // per lane; rows past Nq read the last row, and their elements are
    // masked). Full halves are copied from scalar bases with one per-lane
    // offset (no per-copy address arithmetic); a ragged last tile clamps its
    // rows.
    const uint32_t cpoff = stage_lane_offset<D, kWaves / 2>(wave & 3, lane);
    auto stage_half = [&](int r, int it, int h) {
        size_t rb;
        int t;
        step_rows(it, rb, t);
        const int r0 = t * kQT + h * 32;
        lds_char* qd = qst(r) + h * 32 * D * 2;
        lds_char* dd = dost(r) + h * 32 * D * 2;
        if (r0 + 32 <= Nq) {
            stage_rows_full<D, 32, kWaves / 2>(p.q + rb * D, qd, r0, cpoff, wave & 3);
            stage_rows_full<D, 32, kWaves / 2>(p.dout + rb * D, dd, r0, cpoff, wave & 3);
        } else {
            stage_rows<D, 32, kWaves / 2>(p.q + rb * D, qd, r0, Nq, wave & 3, lane);
            stage_rows<D, 32, kWaves / 2>(p.dout + rb * D, dd, r0, Nq, wave & 3, lane);
        }
        if ((wave & 3) == 0) {
            const float* src = (lane < 32 ? p.lse2 : p.dr) + rb + min(r0 + (lane & 31), Nq - 1);
            copy4_to_lds(src, (uint32_t)(uintptr_t)rvst(r, h));
        }
    };

    // SPARSE: the bitmap of visible steps (bit it of word it / 64), this
    // workgroup's run of them and the order it walks them in.
    lds_u64* const smap = (lds_u64*)(smem + L::kTotal);
    int nsk = 1;                                        // runs of the key block
    int run_begin = 0, run_pivot = 0, run_end = 0;      // the run: steps [run_begin, run_end)
    // The first visible step in [x, end) (end: none).
    auto next_vis = [&](int x, int end) -> int {
        for (int c = x >> 6; c * 64 < end; ++c) {
            uint64_t u = uniform64(smap[c]);
            if (c == (x >> 6)) u &= ~0ull << (x & 63);
            if (u != 0) return min(end, c * 64 + (int)__builtin_ctzll(u));
        }
        return end;
    };
    if constexpr (SPARSE) {
        const int nw = (n_it + 63) / 64;
        for (int c0 = wave; c0 < nw; c0 += 4 * kWaves) {  // four words per wave in flight
            bool on[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * kWaves, it = c * 64 + lane;
                on[u] = false;
                if (c < nw && it < n_it) {
                    const int iq = fast_div(it, p.fd_G);
                    const int tq = t_hi - iq;
                    on[u] = mask_row(p, b, g * p.G + (it - iq * p.G), tq * kQT / kSparseMaskBlock)[kt] != 0;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * kWaves;
                const uint64_t bits = __builtin_amdgcn_ballot_w64(on[u]);
                if (lane == 0 && c < nw) smap[c] = bits;
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // Visible steps V (lane l counts words l, l + 64, ...), and the step
        // index of visible step k (n_it for k >= V).
        int cnt = 0;
        for (int c = lane; c < nw; c += 64) cnt += __builtin_popcountll(smap[c]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
        const int V = __builtin_amdgcn_readfirstlane(cnt);
        auto kth_visible = [&](int k) -> int {
            int base = 0;
            for (int c0 = 0; c0 < nw; c0 += 64) {
                const int c = c0 + lane;
                const uint64_t w = c < nw ? smap[c] : 0ull;
                const int n = __builtin_popcountll(w);
                int pre = n;  // inclusive prefix over the lanes
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(pre, o);
                    if (lane >= o) pre += y;
                }
                const int total = __builtin_amdgcn_readfirstlane(__shfl(pre, 63));
                if (k < base + total) {
                    const uint64_t hit = uniform64(__builtin_amdgcn_ballot_w64(base + pre > k));
                    const int l = (int)__builtin_ctzll(hit);
                    uint64_t wl = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)(w >> 32), l)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)(uint32_t)w, l));
                    const int rem = k - base - __builtin_amdgcn_readfirstlane(__shfl(pre - n, l));
                    for (int i = 0; i < rem; ++i) wl &= wl - 1;
                    return (c0 + l) * 64 + (int)__builtin_ctzll(wl);
                }
                base += total;
            }
            return n_it;
        };
        // Runs: equal in size, as many as needed for at most kSparseRun
        // visible steps each, but no more than p.nseg; a workgroup past the
        // key block's runs has nothing to do (uniform exit).
        nsk = V <= kSparseRun ? 1 : min(p.nseg, (V + kSparseRun - 1) / kSparseRun);
        if (seg >= nsk) return;
        const int per = (V + nsk - 1) / nsk;
        const int v0 = seg * per, v1 = min(V, v0 + per);
        if (v0 < v1) {
            run_begin = kth_visible(v0);
            const int last = kth_visible(v1 - 1);
            run_end = last + 1;
            // A run that reaches the last query tile is walked from the top
            // down, as the dense walk is, so all such runs (causal or full
            // masks, global columns) read the same tiles together. Any other
            // run starts at its tile t* with the largest t mod P (P: the
            // power of two at least the run's span of tiles) and goes down,
            // wrapping from its lowest tile to its highest: runs that are
            // shifted copies of each other (a local window) then start at
            // tiles with the same t mod P and also read the same Q / dO tiles
            // at about the same time on an XCD, sharing them in L2.
            const int t_top = t_hi - fast_div(run_begin, p.fd_G), t_low = t_hi - fast_div(last, p.fd_G);
            int pg = 1;
            while (pg < t_top - t_low + 1) pg <<= 1;
            const int rtop = t_top & (pg - 1);
            const bool top = t_top == n_qt - 1 || rtop == pg - 1 || t_top - rtop - 1 < t_low;
            const int tstar = top ? t_top : t_top - rtop - 1;
            run_pivot = max(run_begin, (t_hi - tstar) * p.G);
        }
    }
    // SPARSE walk order: the visible steps of [run_pivot, run_end), then
    // those of [run_begin, run_pivot); n_it after the last.
    auto sparse_first = [&]() -> int {
        const int x = next_vis(run_pivot, run_end);
        if (x < run_end) return x;
        const int y = next_vis(run_begin, run_pivot);
        return y < run_pivot ? y : n_it;
    };
    auto sparse_after = [&](int x) -> int {
        if (x >= run_pivot) {
            const int y = next_vis(x + 1, run_end);
            if (y < run_end) return y;
            const int z = next_vis(run_begin, run_pivot);
            return z < run_pivot ? z : n_it;
        }
        const int y = next_vis(x + 1, run_pivot);
        return y < run_pivot ? y : n_it;
    };

    // K / V rows of the workgroup (once).
    stage_rows<D, kKW, kWaves>(kbase, kt_, k0, Nk, wave, lane);
    stage_rows<D, kKW, kWaves>(vbase, vt_, k0, Nk, wave, lane);

    // Operand offsets, kept as one base per read kind (the k-step and dim
    // block offsets differ from it by an xor with a constant): K / V B
    // fragments of this wave's keys, Q / dO rows of its query half in
    // MFMA-row order, transposing reads of its query half.
    const int bkoff0 = tile_off<D>(kb4 * 32 + col, half);
    const int aqoff0 = tile_off<D>(qh * 32 + row_of_mfma_row(col), half);
    int troff0[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) troff0[h] = tr_off<D>(0, h, lane) + qh * 32 * D * 2;

    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }
    const int key = k0 + kb4 * 32 + col;  // this lane's key

    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    // The causal d = 128 kernel keeps this wave's K fragments (the B operand
    // of S = Q K^T, the same for every step) in registers for the whole
    // walk: the S/dP products then read 1.5 KiB per MFMA from LDS instead of
    // 2, with their reads one k-step ahead (two no longer fit). Measured
    // +0.7% on the backward; the other instantiations would spill with it.
    constexpr bool kKInRegs = D == 128 && CAUSAL && !WINDOW && !SPARSE;
    bf16x8 kfrag[KS];
    // S = Q K^T, dP = dO V^T for the wave's query half of the step at ring
    // position r: k-step ks reads Q / dO rows (A) and this wave's K / V rows
    // (B), kLead k-steps ahead of its products.
    auto scores = [&](int r, f32x16& s, f32x16& dp) {
        const lds_char* qs_ = qst(r);
        const lds_char* ds_ = dost(r);
        constexpr int LS = kKInRegs ? 1 : kLead;  // k-steps the reads run ahead
        bf16x8 fa_[KS], fb[KS], fc[KS], fd[KS];
        auto rd = [&](int ks) {
            fa_[ks] = *reinterpret_cast<const lds_bf16x8*>(qs_ + tile_off_ks(aqoff0, ks));
            if constexpr (kKInRegs) fb[ks] = kfrag[ks];
            else fb[ks] = *reinterpret_cast<const lds_bf16x8*>(kt_ + tile_off_ks(bkoff0, ks));
            fc[ks] = *reinterpret_cast<const lds_bf16x8*>(ds_ + tile_off_ks(aqoff0, ks));
            fd[ks] = *reinterpret_cast<const lds_bf16x8*>(vt_ + tile_off_ks(bkoff0, ks));
        };
        const f32x16 zero = {};
#pragma unroll
        for (int ks = 0; ks < LS; ++ks) rd(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + LS < KS) rd(ks + LS);
            s = mfma32(fa_[ks], fb[ks], ks == 0 ? zero : s);
            dp = mfma32(fc[ks], fd[ks], ks == 0 ? zero : dp);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // P = exp2(S * scale * log2 e - LSE) and dS = P (dP - Dr) in bf16, for
    // step it at ring position r. Register r of lane half h holds query
    // 16*(r/8) + 8*h + r%8 of the wave's 32 (tile row qh*32 + that), key =
    // this lane's. Its LSE and Dr values are two runs of 8 floats: four
    // 16-byte reads each.
    auto probs = [&](int r, int it, const f32x16& s, const f32x16& dp, bf16x8 (&pb)[2], bf16x8 (&dsb)[2]) {
        size_t rb;
        int t;
        step_rows(it, rb, t);
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        const lds_f32x4* l2s = (const lds_f32x4*)(rvst(r, qh) + 8 * half);
        const lds_f32x4* drs = (const lds_f32x4*)(rvst(r, qh) + 32 + 8 * half);
        // Masking (by a -inf exponent) only where the wave's 32 queries reach
        // past Nq or, causal, below its last key's first visible query.
        const int qbase = t * kQT + qh * 32;  // the wave's first query of the step
        const int kw0 = k0 + kb4 * 32;        // the wave's first key
        const bool masked = qbase + 31 >= Nq || ((CAUSAL || WINDOW) && kw0 + 31 - shift - right > qbase) ||
                            (WINDOW && kw0 - shift + left < qbase + 31);
        const int qrow0 = qbase + 8 * half;   // query of register 0 in this lane
        auto elementwise = [&](auto msk) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {  // registers 8*hh .. 8*hh+7: one run of 8 queries
                __builtin_amdgcn_sched_barrier(0);
                const f32x4 l2v[2] = {l2s[4 * hh], l2s[4 * hh + 1]};
                const f32x4 drv[2] = {drs[4 * hh], drs[4 * hh + 1]};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int rr = 8 * hh + e;
                    float x = __builtin_fmaf(s[rr], p.scale_log2, -l2v[e >> 2][e & 3]);
                    if constexpr (decltype(msk)::value) {
                        const int qg = qrow0 + 16 * hh + e;
                        x = (qg < Nq && !((CAUSAL || WINDOW) && key > qg + shift + right) &&
                             !(WINDOW && key < qg + shift - left)) ? x : -INFINITY;
                    }
                    const float pr = __builtin_amdgcn_exp2f(x);
                    pb[hh][e] = (__bf16)pr;
                    dsb[hh][e] = (__bf16)(pr * (dp[rr] - drv[e >> 2][e & 3]));
                }
            }
        };
        if (masked) elementwise(std::true_type{});
        else elementwise(std::false_type{});
    };
    // dV^T += dO^T P, dK^T += Q^T dS over the wave's two 16-query slices of
    // the step at ring position r (transposing reads kLead products ahead).
    auto grads = [&](int r, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) {
        __builtin_amdgcn_s_setprio(1);  // the matrix phase: dV/dK, then S/dP of the next step
        const lds_char* qs_ = qst(r);
        const lds_char* ds_ = dost(r);
        constexpr int NP = 2 * DB;
        bf16x8 ta[NP], tb[NP];
        auto rd = [&](int n) {
            ta[n] = read_tr_db<D>(ds_, troff0, n % DB, n / DB);
            tb[n] = read_tr_db<D>(qs_, troff0, n % DB, n / DB);
        };
#pragma unroll
        for (int n = 0; n < kLead; ++n) rd(n);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            if (n + kLead < NP) rd(n + kLead);
            dvacc[n % DB] = mfma32(ta[n], pb[n / DB], dvacc[n % DB]);
            dkacc[n % DB] = mfma32(tb[n], dsb[n / DB], dkacc[n % DB]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto end_slot = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    // Ping-pong over the walk x_0, x_1, ... (dense: every step in order;
    // SPARSE: the run's visible steps in its walk order; n_it ends both).
    // Waves w and w + 4 share a SIMD and the same keys: group A (waves 0-3)
    // takes query half 0 of every step, group B (waves 4-7) half 1.
    // Workgroup barriers cut time into slots, and in every slot one group
    // runs its products while the other runs its elementwise phase (and
    // issues the copies), so each SIMD has MFMA work from one wave and VALU
    // work from the other (step x_j at ring position j & 1):
    //   slot 2j  : A: dV/dK of x_{j-1}, S/dP of x_j | B: P/dS of x_{j-1}; copies half 1 of x_j
    //   slot 2j+1: A: P/dS of x_j; copies half 0 of x_{j+1} | B: dV/dK of x_{j-1}, S/dP of x_j
    // Half h of a ring position is last read by dV/dK of x_{j-1} in slot
    // 2j+h and refilled with half h of x_{j+1} in slot 2j+1+h, which it is
    // first read after (slot 2j+2+h). Every barrier waits for the copies.
    // Each wave accumulates the same products in the same order as without
    // the ping-pong; only their timing differs.
    bool walked = false;  // SPARSE: the run has a visible step
    {
        int cur = SPARSE ? sparse_first() : 0;  // x_j
        const bool grp_b = wave >= kWaves / 2;
        if (cur < n_it) walked = true;
        if (!grp_b && cur < n_it) stage_half(0, cur, 0);  // half 0 of x_0
        end_slot();
        if constexpr (kKInRegs) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kfrag[ks] = *reinterpret_cast<const lds_bf16x8*>(kt_ + tile_off_ks(bkoff0, ks));
        }
        f32x16 s, dp;
        bf16x8 pb[2], dsb[2];
        int nxt = cur < n_it ? (SPARSE ? sparse_after(cur) : cur + 1) : n_it;  // x_{j+1}
        if (!grp_b) {
            __builtin_amdgcn_s_setprio(1);
            if (cur < n_it) scores(0, s, dp);  // slot 0
            for (int j = 0; cur < n_it; ++j) {
                end_slot();
                __builtin_amdgcn_s_setprio(0);  // the elementwise phase
                if (nxt < n_it) stage_half(j + 1, nxt, 0);  // slot 2j+1
                probs(j, cur, s, dp, pb, dsb);
                end_slot();
                grads(j, pb, dsb);  // slot 2j+2
                if (nxt < n_it) scores(j + 1, s, dp);
                cur = nxt;
                if (nxt < n_it) nxt = SPARSE ? sparse_after(nxt) : nxt + 1;
            }
            __builtin_amdgcn_s_setprio(0);
            end_slot();  // A has no work in B's last slot
        } else {
            if (cur < n_it) stage_half(0, cur, 1);  // slot 0
            end_slot();
            __builtin_amdgcn_s_setprio(1);
            if (cur < n_it) scores(0, s, dp);  // slot 1
            for (int j = 0; cur < n_it; ++j) {
                end_slot();
                __builtin_amdgcn_s_setprio(0);  // the elementwise phase
                if (nxt < n_it) stage_half(j + 1, nxt, 1);  // slot 2j+2
                probs(j, cur, s, dp, pb, dsb);
                end_slot();
                grads(j, pb, dsb);  // slot 2j+3
                if (nxt < n_it) scores(j + 1, s, dp);
                cur = nxt;
                if (nxt < n_it) nxt = SPARSE ? sparse_after(nxt) : nxt + 1;
            }
            __builtin_amdgcn_s_setprio(0);
        }
    }

    // Sum the two query halves (waves w and w + 4), then store.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    lds_float* red = (lds_float*)smem + kb4 * (2 * DB * 16 * 64);
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                red[(db * 16 + r) * 64 + lane] = dkacc[db][r];
                red[((DB + db) * 16 + r) * 64 + lane] = dvacc[db][r];
            }
    }
    __syncthreads();
    if (SPARSE && p.nseg > 1 && seg == 0 && tid == 0) p.seg_count[(size_t)unit * p.n_ktiles + kt] = (uint32_t)nsk;
    if (SPARSE && nsk > 1) {  // one run of several: the fp32 partial (unscaled) and its flag
        const size_t slot = ((size_t)unit * p.n_ktiles + kt) * p.nseg + seg;
        if (tid == 0) p.seg_flags[slot] = walked ? 1u : 0u;
        if (qh == 0 && walked) {
            // Registers 4*q4 .. 4*q4+3 of block db (q = 4*db + q4) as one
            // 16-byte vector per lane: [wave][q][lane][4] floats.
            f32x4* pk = (f32x4*)(p.partial + slot * (2 * kKW * D)) + kb4 * (DB * 4 * 64) + lane;
            f32x4* pv = pk + kKW * D / 4;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    f32x4 xk, xv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * q4 + e;
                        xk[e] = dkacc[db][r] + red[(db * 16 + r) * 64 + lane];
                        xv[e] = dvacc[db][r] + red[((DB + db) * 16 + r) * 64 + lane];
                    }
                    pk[(db * 4 + q4) * 64] = xk;
                    pv[(db * 4 + q4) * 64] = xv;
                }
        }
        return;
    }
    if (qh == 0 && key < Nk) {
        const size_t krow = ((size_t)b * p.Hkv + g) * Nk + key;
        uint16_t* dkp = p.dk + krow * D;
        uint16_t* dvp = p.dv + krow * D;
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 kv4, vv4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r4 * 4 + e;
                    kv4[e] = (__bf16)((dkacc[db][r] + red[(db * 16 + r) * 64 + lane]) * p.scale);
                    vv4[e] = (__bf16)(dvacc[db][r] + red[((DB + db) * 16 + r) * 64 + lane]);
                }
                *reinterpret_cast<bf16x4*>(dkp + db * 32 + r4 * 8 + half * 4) = kv4;
                *reinterpret_cast<bf16x4*>(dvp + db * 32 + r4 * 8 + half * 4) = vv4;
            }
    }
}

// ---- dK, dV of key blocks whose block-sparse walk was cut into runs ---------
// One workgroup per key block of 128 keys: the runs' fp32 partials summed in
// run order (runs without a visible step skipped), dK scaled, both rounded to
// bf16. Thread (w, lane) holds the values wave w of fa_bwd_dkdv held: key
// 32*w + lane%32, and the same register order. Key blocks walked by one
// workgroup were written by it and are skipped.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_dkdv_combine(BwdParams p) {
    constexpr int DB = D / 32;
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int kb4 = tid >> 6;
    const int n_units = p.B * p.Hkv;
    const int unit = blockIdx.x % n_units, kt = blockIdx.x / n_units;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int k0 = kt * kKW, Nk = p.Nk;
    const int nsk = (int)p.seg_count[(size_t)unit * p.n_ktiles + kt];
    if (nsk <= 1) return;
    f32x4 dk[DB * 4], dv[DB * 4];  // register 4*q + e of fa_bwd_dkdv's block q / 4 in dk[q][e]
#pragma unroll
    for (int q = 0; q < DB * 4; ++q) dk[q] = dv[q] = f32x4{};
    const size_t slot0 = ((size_t)unit * p.n_ktiles + kt) * p.nseg;
    for (int sg = 0; sg < nsk; ++sg) {
        if (p.seg_flags[slot0 + sg] == 0) continue;
        const f32x4* pk = (const f32x4*)(p.partial + (slot0 + sg) * (2 * kKW * D)) + kb4 * (DB * 4 * 64) + lane;
        const f32x4* pv = pk + kKW * D / 4;
        f32x4 xk[DB * 4], xv[DB * 4];
#pragma unroll
        for (int q = 0; q < DB * 4; ++q) {
            xk[q] = pk[q * 64];
            xv[q] = pv[q * 64];
        }
#pragma unroll
        for (int q = 0; q < DB * 4; ++q) {
            dk[q] += xk[q];
            dv[q] += xv[q];
        }
    }
    const int key = k0 + kb4 * 32 + col;
    if (key >= Nk) return;
    const size_t krow = ((size_t)b * p.Hkv + g) * Nk + key;
    uint16_t* dkp = p.dk + krow * D;
    uint16_t* dvp = p.dv + krow * D;
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 kv4, vv4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kv4[e] = (__bf16)(dk[db * 4 + r4][e] * p.scale);
                vv4[e] = (__bf16)dv[db * 4 + r4][e];
            }
            *reinterpret_cast<bf16x4*>(dkp + db * 32 + r4 * 8 + half * 4) = kv4;
            *reinterpret_cast<bf16x4*>(dvp + db * 32 + r4 * 8 + half * 4) = vv4;
        }
}

int pow2_divisor_upto8(int G) {
    int h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

template <int D, bool CAUSAL, bool WINDOW, bool SPARSE>
void launch_dq(const BwdParams& p, long long grid, hipStream_t stream) {
    if (trace_on())
        trace("fa_bwd_dq<d=%d, causal=%d, window=%d, sparse=%d> grid=%lld block=%d", D, (int)CAUSAL, (int)WINDOW,
              (int)SPARSE, grid, kThreads);
    hipLaunchKernelGGL((fa_bwd_dq<D, CAUSAL, WINDOW, SPARSE>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
}

template <int D, bool CAUSAL, bool WINDOW, bool SPARSE>
void launch_dkdv(const BwdParams& p, long long grid, hipStream_t stream) {
    if (trace_on())
        trace("fa_bwd_dkdv<d=%d, causal=%d, window=%d, sparse=%d> grid=%lld block=%d", D, (int)CAUSAL, (int)WINDOW,
              (int)SPARSE, grid, kThreads);
    hipLaunchKernelGGL((fa_bwd_dkdv<D, CAUSAL, WINDOW, SPARSE>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
}

// The WINDOW kernels serve a window (causal folded into its right bound),
// the SPARSE ones a block mask (causal or not); the two never combine.
template <int D>
hipError_t launch_d(BwdParams& p, bool causal, bool window, bool sparse, hipStream_t stream) {
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    if (rows > 0) {
        const long long blocks = (rows + (256 / (D / 8)) - 1) / (256 / (D / 8));
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        if (trace_on()) trace("fa_bwd_pre<d=%d> grid=%lld block=256", D, blocks);
        hipLaunchKernelGGL((fa_bwd_pre<D>), dim3((unsigned)blocks), dim3(256), 0, stream, p, rows);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const long long gq = (long long)p.n_units * p.n_qtiles;
    if (gq > 0) {
        if (window) launch_dq<D, false, true, false>(p, gq, stream);
        else if (sparse) causal ? launch_dq<D, true, false, true>(p, gq, stream)
                                : launch_dq<D, false, false, true>(p, gq, stream);
        else if (causal) launch_dq<D, true, false, false>(p, gq, stream);
        else launch_dq<D, false, false, false>(p, gq, stream);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const long long gk = (long long)p.B * p.Hkv * p.n_ktiles;
    if (gk > 0) {
        if (window) launch_dkdv<D, false, true, false>(p, gk, stream);
        else if (sparse) causal ? launch_dkdv<D, true, false, true>(p, gk * p.nseg, stream)
                                : launch_dkdv<D, false, false, true>(p, gk * p.nseg, stream);
        else if (causal) launch_dkdv<D, true, false, false>(p, gk, stream);
        else launch_dkdv<D, false, false, false>(p, gk, stream);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        if (sparse && p.nseg > 1) {
            if (trace_on()) trace("fa_bwd_dkdv_combine<d=%d> grid=%lld block=256", D, gk);
            hipLaunchKernelGGL((fa_bwd_dkdv_combine<D>), dim3((unsigned)gk), dim3(256), 0, stream, p);
            if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        }
    }
    return hipSuccess;
}

}  // namespace

SparseBwdPlan sparse_backward_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    SparseBwdPlan pl{1, 0, 0, 0, (size_t)B * Hq * Nq * 8};  // one run: the per-row values only
    const size_t rows = (pl.bytes + 255) / 256 * 256;
    // Runs per key block: enough that a key block every query block sees
    // (G * query tiles steps) is cut into runs of at most kSparseRun steps,
    // but at most ceil(16 / (B * Hkv)): with few (batch, K/V head) pairs a whole
    // column is far longer than the grid's average work per CU, with many
    // it is not (and the partials, nseg * B * Hkv * Nk * d * 8 bytes, stay
    // near 16 * Nk * d * 8).
    const long long n_it = (long long)(Hq / Hkv) * ((Nq + kQT - 1) / kQT);
    const long long bh = (long long)B * Hkv;
    const long long cap = std::max(1LL, (16LL + bh - 1) / bh);
    const long long nseg = std::min(cap, std::max(1LL, (n_it + kSparseRun - 1) / kSparseRun));
    if (nseg <= 1) return pl;
    pl.nseg = (int)nseg;
    const size_t kblocks = (size_t)bh * ((Nk + kKW - 1) / kKW);
    const size_t slots = kblocks * nseg;
    pl.partial_offset = rows;
    pl.flags_offset = rows + slots * 2 * kKW * d * sizeof(float);
    pl.counts_offset = pl.flags_offset + slots * sizeof(uint32_t);
    pl.bytes = pl.counts_offset + kblocks * sizeof(uint32_t);
    return pl;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    BwdParams p = {};
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.o = static_cast<const uint16_t*>(a.o);
    p.dout = static_cast<const uint16_t*>(a.dout);
    p.lse = a.lse;
    p.dq = static_cast<uint16_t*>(a.dq);
    p.dk = static_cast<uint16_t*>(a.dk);
    p.dv = static_cast<uint16_t*>(a.dv);
    p.dr = static_cast<float*>(a.workspace);
    p.lse2 = p.dr + (size_t)a.B * a.Hq * a.Nq;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
    p.G = a.Hq / a.Hkv;
    p.heads_per_wg = pow2_divisor_upto8(p.G);
    p.qblocks_per_wg = kWaves / p.heads_per_wg;
    p.n_hsub = p.G / p.heads_per_wg;
    p.n_qtiles = (a.Nq + kRows * p.qblocks_per_wg - 1) / (kRows * p.qblocks_per_wg);
    p.n_units = a.B * a.Hkv * p.n_hsub;
    p.n_ktiles = (a.Nk + kKW - 1) / kKW;
    p.qb_log2 = 0;
    while ((1 << p.qb_log2) < p.qblocks_per_wg) ++p.qb_log2;
    p.fd_units = make_fastdiv(p.n_units);
    p.fd_hsub = make_fastdiv(p.n_hsub);
    p.fd_hkv = make_fastdiv(a.Hkv);
    p.fd_kvunits = make_fastdiv(a.B * a.Hkv);
    p.fd_G = make_fastdiv(p.G);
    p.fd_nseg = make_fastdiv(1);
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    if ((long long)p.n_units * p.n_qtiles > 0x7fffffffLL || (long long)a.B * a.Hkv * p.n_ktiles > 0x7fffffffLL)
        return hipErrorInvalidValue;
    // A window runs the WINDOW kernels, with causal folded into a right bound of 0.
    const bool window = a.window_left >= 0 || (!a.causal && a.window_right >= 0);
    p.win_left = a.window_left;
    p.win_right = a.causal ? 0 : a.window_right;
    const bool sparse = a.block_mask != nullptr;
    if (sparse) {
        p.bmask = a.block_mask;
        p.bm_sb = a.mask_stride_b;
        p.bm_sh = a.mask_stride_h;
        p.n_kb = (a.Nk + kSparseMaskBlock - 1) / kSparseMaskBlock;
        if (window || p.n_kb > kSparseMaxKeyBlocks) return hipErrorInvalidValue;
        const SparseBwdPlan pl = sparse_backward_plan(a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d);
        if ((long long)p.G * ((a.Nq + kQT - 1) / kQT) > kSparseMaxSteps) return hipErrorInvalidValue;
        p.nseg = pl.nseg;
        p.fd_nseg = make_fastdiv(pl.nseg);
        if (pl.nseg > 1) {
            p.partial = (float*)((char*)a.workspace + pl.partial_offset);
            p.seg_flags = (uint32_t*)((char*)a.workspace + pl.flags_offset);
            p.seg_count = (uint32_t*)((char*)a.workspace + pl.counts_offset);
        }
        if ((long long)a.B * a.Hkv * p.n_ktiles * p.nseg > 0x7fffffffLL) return hipErrorInvalidValue;
    }
    return a.d == 128 ? launch_d<128>(p, a.causal != 0, window, sparse, stream)
                      : launch_d<64>(p, a.causal != 0, window, sparse, stream);
}

}  // namespace fa
