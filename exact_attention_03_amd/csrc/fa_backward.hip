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

#include <type_traits>

#include "fa_kernels.h"
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
    // Sliding window (WINDOW kernels): query i at key position p = i + Nk - Nq
    // sees keys [p - win_left, p + win_right]; a negative bound is none.
    int win_left, win_right;
    float scale, scale_log2;
};

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
template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq(BwdParams p) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int SB = kKT * D * 2;  // bytes of one K or V stage
    // K stages: tile j is read until two slots after its scores (by the
    // products dQ^T += K^T dS^T), so the ring needs three; it has four, as a
    // stage index of j % 3 made the compiler keep per-stage address vectors
    // (and spill) where j & 3 costs nothing. Two V stages.
    __shared__ __attribute__((aligned(1024))) char smem_raw[6 * SB];
    lds_char* smem = (lds_char*)smem_raw;
    auto kst = [&](int j) { return smem + (j & 3) * SB; };
    auto vst = [&](int j) { return smem + (4 + (j & 1)) * SB; };

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int id = blockIdx.x;
    const int unit = id % p.n_units;
    int qt = id / p.n_units;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest first
    const int hsub = unit % p.n_hsub;
    const int g = (unit / p.n_hsub) % p.Hkv;
    const int b = unit / (p.n_hsub * p.Hkv);
    const int rows_q = kRows * p.qblocks_per_wg;
    const int qtile0 = qt * rows_q;
    const int head = g * p.G + hsub * p.heads_per_wg + wave / p.qblocks_per_wg;
    const int q0 = qtile0 + (wave % p.qblocks_per_wg) * kRows;
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
    // S^T and dP^T: product n uses the K and V rows of 32-key block n / KS
    // at k-step n % KS, read kLead products ahead.
    auto scores = [&](int j) {
        typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
        const lds_char* ks_ = kst(j);
        const lds_char* vs_ = vst(j);
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
    // dS^T = P^T (dP^T - Dr); register r of block kb2 holds key
    // 32*kb2 + 16*(r/8) + 8*half + r%8 of the tile. Masked keys get a -inf
    // exponent (a select, no per-element control flow).
    auto elementwise = [&](int j) {
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int kb2 = 0; kb2 < kKT / 32; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j * kKT + kb2 * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
                float x = __builtin_fmaf(s[kb2][r], p.scale_log2, -lse2);
                x = (key <= lim && (!WINDOW || key >= lo)) ? x : -INFINITY;
                const float pr = __builtin_amdgcn_exp2f(x);
                dsb[kb2 * 2 + (r >> 3)][r & 7] = (__bf16)(pr * (dp[kb2][r] - dr));
            }
        // dS is complete here: keeps the work in this phase instead of letting
        // the compiler sink it into the next matrix phase.
#pragma unroll
        for (int t = 0; t < kKT / 16; ++t) asm volatile("" : : "v"(dsb[t]));
    };
    // dQ^T += K^T dS^T over the tile's four 16-key slices (K^T read kLead
    // products ahead). Raises the wave's priority for its matrix phase.
    auto products = [&](int j) {
        __builtin_amdgcn_s_setprio(1);
        const lds_char* ks_ = kst(j);
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
    if (nt > t0) {
        stage_rows<D, kKT, kWaves>(kb, kst(t0), t0 * kKT, Nk, wave, lane);
        stage_rows<D, kKT, kWaves>(vb, vst(t0), t0 * kKT, Nk, wave, lane);
        if (t0 + 1 < nt) {
            stage_rows<D, kKT, kWaves>(kb, kst(t0 + 1), (t0 + 1) * kKT, Nk, wave, lane);
            stage_rows<D, kKT, kWaves>(vb, vst(t0 + 1), (t0 + 1) * kKT, Nk, wave, lane);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
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
        auto end_even_slot = [&](int j) {  // copies for slot 2j+3 issued after this
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const int j2 = j + 2;
            if (wave < kWaves / 2 && j2 < nt) {
                if ((j2 + 1) * kKT <= Nk) {
                    stage_rows_full<D, kKT, kWaves / 2>(kb, kst(j2), j2 * kKT, cpoff, wave);
                    stage_rows_full<D, kKT, kWaves / 2>(vb, vst(j2), j2 * kKT, cpoff, wave);
                } else {
                    int l = lane;
                    asm volatile("" : "+v"(l));
                    stage_rows<D, kKT, kWaves / 2>(kb, kst(j2), j2 * kKT, Nk, wave, l);
                    stage_rows<D, kKT, kWaves / 2>(vb, vst(j2), j2 * kKT, Nk, wave, l);
                }
            }
        };
        // Each group's loop body is scores(j), elementwise(j), products(j)
        // with the barriers placed for its offset, so only the accumulators
        // and the fragments of Q and dO live across iterations.
        if (wave < kWaves / 2) {
            for (int j = t0; j < nt; ++j) {
                scores(j);            // slot 2j-1 (slot 0 for the first tile)
                if (j > t0) end_odd_slot();
                elementwise(j);       // slot 2j
                end_even_slot(j);
                products(j);          // slot 2j+1
            }
            end_odd_slot();
        } else {
            for (int j = t0; j < nt; ++j) {
                scores(j);            // slot 2j
                end_even_slot(j);
                elementwise(j);       // slot 2j+1
                end_odd_slot();
                products(j);          // slot 2j+2
            }
        }
        __builtin_amdgcn_s_setprio(0);
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

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv(BwdParams p) {
    using L = DkdvLds<D>;
    constexpr int KS = D / 16, DB = D / 32;
    __shared__ __attribute__((aligned(1024))) char smem_raw[L::kTotal];
    lds_char* smem = (lds_char*)smem_raw;
    lds_char* kt_ = smem;
    lds_char* vt_ = smem + L::kKV;
    auto qst = [&](int j) { return smem + 2 * L::kKV + (j & 1) * L::kQ; };
    auto dost = [&](int j) { return smem + 2 * L::kKV + (2 + (j & 1)) * L::kQ; };
    typedef __attribute__((address_space(3))) float lds_float;
    auto lsest = [&](int j) { return (lds_float*)(smem + 2 * L::kKV + 4 * L::kQ + (j & 1) * L::kRowVals); };
    auto drst = [&](int j) { return (lds_float*)(smem + 2 * L::kKV + 4 * L::kQ + (2 + (j & 1)) * L::kRowVals); };

    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb4 = wave & 3;   // this wave's 32-key block
    const int qh = wave >> 2;   // this wave's query half of each tile

    const int id = blockIdx.x;
    const int n_units = p.B * p.Hkv;
    const int unit = id % n_units;
    const int kt = id / n_units;  // heaviest (earliest keys) first under the causal mask
    const int b = unit / p.Hkv, g = unit % p.Hkv;
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
        const int hh = it % p.G;
        t = t_hi - it / p.G;
        rowbase = ((size_t)b * p.Hq + g * p.G + hh) * Nq;
    };
    // Copies of step it: the Q and dO rows (all waves), and the step's 64
    // LSE (exp2 units) and Dr values (waves 0 and 1, 4 bytes per lane; rows
    // past Nq read the last row, and their elements are masked).
    // Full tiles are copied from scalar bases with one per-lane offset (no
    // per-copy address arithmetic); a ragged last tile clamps its rows.
    const uint32_t cpoff = stage_lane_offset<D, kWaves>(wave, lane);
    auto stage_step = [&](int it) {
        size_t rb;
        int t;
        step_rows(it, rb, t);
        if ((t + 1) * kQT <= Nq) {
            stage_rows_full<D, kQT, kWaves>(p.q + rb * D, qst(it), t * kQT, cpoff, wave);
            stage_rows_full<D, kQT, kWaves>(p.dout + rb * D, dost(it), t * kQT, cpoff, wave);
        } else {
            stage_rows<D, kQT, kWaves>(p.q + rb * D, qst(it), t * kQT, Nq, wave, lane);
            stage_rows<D, kQT, kWaves>(p.dout + rb * D, dost(it), t * kQT, Nq, wave, lane);
        }
        if (wave < 2) {
            const float* src = (wave == 0 ? p.lse2 : p.dr) + rb + min(t * kQT + lane, Nq - 1);
            copy4_to_lds(src, (uint32_t)(uintptr_t)(wave == 0 ? lsest(it) : drst(it)));
        }
    };

    // K / V rows of the workgroup (once), and the first step.
    stage_rows<D, kKW, kWaves>(kbase, kt_, k0, Nk, wave, lane);
    stage_rows<D, kKW, kWaves>(vbase, vt_, k0, Nk, wave, lane);
    if (n_it > 0) stage_step(0);

    // Operand offsets: K^T / V^T B fragments of this wave's keys, Q / dO rows
    // of its query half in MFMA-row order, transposing reads.
    int bkoff[KS], aqoff[KS], troff[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bkoff[ks] = tile_off<D>(kb4 * 32 + col, 2 * ks + half);
        aqoff[ks] = tile_off<D>(qh * 32 + row_of_mfma_row(col), 2 * ks + half);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) troff[db][h] = tr_off<D>(db, h, lane) + qh * 32 * D * 2;

    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }
    const int key = k0 + kb4 * 32 + col;  // this lane's key

    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    for (int it = 0; it < n_it; ++it) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // step it staged; every wave is done with step it - 1
        if (it + 1 < n_it) stage_step(it + 1);
        size_t rb;
        int t;
        step_rows(it, rb, t);
        const lds_char* qs_ = qst(it);
        const lds_char* ds_ = dost(it);
        // S = Q K^T, dP = dO V^T: k-step ks reads Q / dO rows (A) and this
        // wave's K / V rows (B), kLead k-steps ahead of its products.
        f32x16 s, dp;
        {
            bf16x8 fa_[KS], fb[KS], fc[KS], fd[KS];
            auto rd = [&](int ks) {
                fa_[ks] = *reinterpret_cast<const lds_bf16x8*>(qs_ + aqoff[ks]);
                fb[ks] = *reinterpret_cast<const lds_bf16x8*>(kt_ + bkoff[ks]);
                fc[ks] = *reinterpret_cast<const lds_bf16x8*>(ds_ + aqoff[ks]);
                fd[ks] = *reinterpret_cast<const lds_bf16x8*>(vt_ + bkoff[ks]);
            };
            const f32x16 zero = {};
#pragma unroll
            for (int ks = 0; ks < kLead; ++ks) rd(ks);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + kLead < KS) rd(ks + kLead);
                s = mfma32(fa_[ks], fb[ks], ks == 0 ? zero : s);
                dp = mfma32(fc[ks], fd[ks], ks == 0 ? zero : dp);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // Register r of lane half h holds query 16*(r/8) + 8*h + r%8 of the
        // wave's 32 (tile row qh*32 + that), key = this lane's. Its LSE and
        // Dr values are two runs of 8 floats: four 16-byte reads each.
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
        const lds_f32x4* l2s = (const lds_f32x4*)(lsest(it) + qh * 32 + 8 * half);
        const lds_f32x4* drs = (const lds_f32x4*)(drst(it) + qh * 32 + 8 * half);
        // Masking (by a -inf exponent) only where the wave's 32 queries reach
        // past Nq or, causal, below its last key's first visible query.
        const int qbase = t * kQT + qh * 32;  // the wave's first query of the step
        const int kw0 = k0 + kb4 * 32;        // the wave's first key
        const bool masked = qbase + 31 >= Nq || ((CAUSAL || WINDOW) && kw0 + 31 - shift - right > qbase) ||
                            (WINDOW && kw0 - shift + left < qbase + 31);
        const int qrow0 = qbase + 8 * half;   // query of register 0 in this lane
        bf16x8 pb[2], dsb[2];
        auto elementwise = [&](auto msk) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {  // registers 8*hh .. 8*hh+7: one run of 8 queries
                __builtin_amdgcn_sched_barrier(0);  // reads issued here, after the products above
                const f32x4 l2v[2] = {l2s[4 * hh], l2s[4 * hh + 1]};
                const f32x4 drv[2] = {drs[4 * hh], drs[4 * hh + 1]};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * hh + e;
                    float x = __builtin_fmaf(s[r], p.scale_log2, -l2v[e >> 2][e & 3]);
                    if constexpr (decltype(msk)::value) {
                        const int qg = qrow0 + 16 * hh + e;
                        x = (qg < Nq && !((CAUSAL || WINDOW) && key > qg + shift + right) &&
                         !(WINDOW && key < qg + shift - left)) ? x : -INFINITY;
                    }
                    const float pr = __builtin_amdgcn_exp2f(x);
                    pb[hh][e] = (__bf16)pr;
                    dsb[hh][e] = (__bf16)(pr * (dp[r] - drv[e >> 2][e & 3]));
                }
            }
        };
        if (masked) elementwise(std::true_type{});
        else elementwise(std::false_type{});
        // dV^T += dO^T P, dK^T += Q^T dS over the wave's two 16-query slices
        // (transposing reads kLead products ahead).
        {
            constexpr int NP = 2 * DB;
            bf16x8 ta[NP], tb[NP];
            auto rd = [&](int n) {
                ta[n] = read_tr<D>(ds_, troff, n % DB, n / DB);
                tb[n] = read_tr<D>(qs_, troff, n % DB, n / DB);
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

int pow2_divisor_upto8(int G) {
    int h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

template <int D>
hipError_t launch_d(BwdParams& p, bool causal, bool window, hipStream_t stream) {
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
        if (trace_on())
            trace("fa_bwd_dq<d=%d, causal=%d, window=%d> grid=%lld block=%d", D, (int)(causal && !window),
                  (int)window, gq, kThreads);
        if (window) hipLaunchKernelGGL((fa_bwd_dq<D, false, true>), dim3((unsigned)gq), dim3(kThreads), 0, stream, p);
        else if (causal) hipLaunchKernelGGL((fa_bwd_dq<D, true, false>), dim3((unsigned)gq), dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((fa_bwd_dq<D, false, false>), dim3((unsigned)gq), dim3(kThreads), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const long long gk = (long long)p.B * p.Hkv * p.n_ktiles;
    if (gk > 0) {
        if (trace_on())
            trace("fa_bwd_dkdv<d=%d, causal=%d, window=%d> grid=%lld block=%d", D, (int)(causal && !window),
                  (int)window, gk, kThreads);
        if (window) hipLaunchKernelGGL((fa_bwd_dkdv<D, false, true>), dim3((unsigned)gk), dim3(kThreads), 0, stream, p);
        else if (causal) hipLaunchKernelGGL((fa_bwd_dkdv<D, true, false>), dim3((unsigned)gk), dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((fa_bwd_dkdv<D, false, false>), dim3((unsigned)gk), dim3(kThreads), 0, stream, p);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    return hipSuccess;
}

}  // namespace

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
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    if ((long long)p.n_units * p.n_qtiles > 0x7fffffffLL || (long long)a.B * a.Hkv * p.n_ktiles > 0x7fffffffLL)
        return hipErrorInvalidValue;
    // A window runs the WINDOW kernels, with causal folded into a right bound of 0.
    const bool window = a.window_left >= 0 || (!a.causal && a.window_right >= 0);
    p.win_left = a.window_left;
    p.win_right = a.causal ? 0 : a.window_right;
    return a.d == 128 ? launch_d<128>(p, a.causal != 0, window, stream) : launch_d<64>(p, a.causal != 0, window, stream);
}

}  // namespace fa
