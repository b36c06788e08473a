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
//     two waves per SIMD (each fits in 256 registers, so the MFMA
//     accumulators stay in VGPRs and one wave's softmax can run while the
//     other wave's MFMAs occupy the matrix unit). A row block is 32
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
//     free of bank conflicts. Two LDS stages let the loads of tile j+1
//     overlap the math of tile j.
//   * Lazy rescaling: the running maximum used as the softmax reference is
//     only moved when some row's tile maximum exceeds it by more than 2^8 in
//     exp2 units. The reference cancels exactly between O and the row sum, so
//     the result is unchanged while most tiles skip the O rescale.
//   * Grid: one workgroup per (batch, K/V head, head subset, query tile).
//     Query tiles are issued heaviest-first for causal masks, and when there
//     are a multiple of 8 K/V units, all tiles of one K/V head go to one XCD
//     (workgroups are dealt round-robin to the 8 XCDs) so they share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
#ifndef FA_PREFILL_BN
#define FA_PREFILL_BN 64
#endif
constexpr int kBN = FA_PREFILL_BN;  // keys per K/V tile
constexpr int kNKB = kBN / 32;      // 32-key blocks per tile
constexpr int kBlockRows = 32;      // queries per row block
constexpr int kBlocksPerWG = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // exp2 units the reference may lag behind the max

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
    int causal;
    float scale_log2;    // scale * log2(e)
    float scale;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// XOR swizzle of the 16-byte chunks of a staged K or V row. It is a
// bijection on the row's chunks; for 16 consecutive rows read at one chunk
// (K operand) and for 4 consecutive rows x 4 consecutive chunks (transposing
// V reads) every 16-lane phase lands on distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
// Byte offset of logical 16-byte chunk `c` of row `r` in a staged tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) { return r * (D * 2) + ((c ^ swz<D>(r)) << 4); }

// Key held by MFMA row index i of a 32-key block (see the file header).
__device__ __forceinline__ int key_of_row(int i) {
    int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
    return ((a >> 1) << 4) + (h << 3) + ((a & 1) << 2) + b;
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct Stage {
    static constexpr int kBytesK = kBN * D * 2;
    static constexpr int kBytesV = kBN * D * 2;
    static constexpr int kBytes = kBytesK + kBytesV;
    static constexpr int kInstPerWave = kBytesK / 1024 / kWaves;  // 1 KiB per wave instruction
};

// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; lds_base is wave-uniform and goes through M0,
// which needs one wait state before the copy reads it).
// Issued from asm so the compiler does not make later reads of *other* LDS
// stages wait for this copy; the tile loop waits for it explicitly
// (s_waitcnt vmcnt) before the barrier that publishes the stage.
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_base) : "memory", "m0");
}

// Enqueue the direct global->LDS copy of K/V tile rows [j0, j0+64) into one
// stage. Rows past Nk are clamped to the last row: they are masked out of
// the scores (K) and meet zero weights (V), and stay finite.
template <int D>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ kbase, const uint16_t* __restrict__ vbase,
                                           lds_char* kst, lds_char* vst, int j0, int Nk, int wave, int lane) {
    constexpr int RB = D * 2;          // bytes per row
    constexpr int RPI = 1024 / RB;     // rows per wave instruction
    const int uw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int n = 0; n < Stage<D>::kInstPerWave; ++n) {
        const int blk = n * kWaves + uw;              // which 1 KiB of the tile
        const int r = blk * RPI + lane / (RB / 16);
        const int phys = lane % (RB / 16);
        const int c = phys ^ swz<D>(r);
        const int key = min(j0 + r, Nk - 1);
        const size_t goff = (size_t)key * D + c * 8;
        copy16_to_lds(kbase + goff, (uint32_t)(uintptr_t)(kst + blk * 1024));
        copy16_to_lds(vbase + goff, (uint32_t)(uintptr_t)(vst + blk * 1024));
    }
}

// A operand of O^T += V^T P^T for dim block db and 16-key slice t: dims
// 32*db + lane%32, keys 16*t + 8*(lane/32) .. +7, from two transposing reads.
template <int D>
__device__ __forceinline__ bf16x8 read_vt(const lds_char* vst, int db, int t, int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int dim = db * 32 + 16 * (G & 1) + 4 * (j & 3);
    const int key = 16 * t + 8 * (G >> 1) + (j >> 2);
    const int chunk = dim >> 3, within = (dim & 7) * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vst + tile_off<D>(key, chunk) + within));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vst + tile_off<D>(key + 4, chunk) + within));
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Value of x in lane l^32 (the other 32-lane half).
__device__ __forceinline__ float other_half(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    int lane = __lane_id();
    return __uint_as_float(lane < 32 ? s[1] : s[0]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdParams p) {
    constexpr int KS = D / 16;   // 16-dim k-steps of Q K^T
    constexpr int DB = D / 32;   // 32-dim blocks of O^T
    __shared__ __attribute__((aligned(1024))) char smem_raw[2 * Stage<D>::kBytes];
    lds_char* smem = (lds_char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;

    // ---- workgroup -> (unit, query tile) ----
    int unit, qt;
    {
        const int id = blockIdx.x;
        if (p.xcd_affine) {
            const int xcd = id & 7, k = id >> 3;
            const int ux = p.n_units >> 3;  // units per XCD
            unit = xcd + 8 * (k % ux);
            qt = k / ux;
        } else {
            unit = id % p.n_units;
            qt = id / p.n_units;
        }
        if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest first
    }
    const int hsub = unit % p.n_hsub;
    const int g = (unit / p.n_hsub) % p.Hkv;
    const int b = unit / (p.n_hsub * p.Hkv);
    const int rows_q = kBlockRows * p.qblocks_per_wg;  // queries per tile
    const int qtile0 = qt * rows_q;

    // ---- this wave's row block: 32 queries of one head ----
    const int head = g * p.G + hsub * p.heads_per_wg + wave / p.qblocks_per_wg;
    const int q0 = qtile0 + (wave % p.qblocks_per_wg) * kBlockRows;
    const int shift = p.Nk - p.Nq;  // causal: key j visible from query i iff j <= i + shift

    // Key range of the workgroup and of this wave.
    int wg_kend = p.Nk, wave_kend = p.Nk, wave_kmask = p.Nk;
    if (CAUSAL) {
        const int wg_qlast = min(p.Nq, qtile0 + rows_q) - 1;
        wg_kend = max(0, min(p.Nk, wg_qlast + 1 + shift));
        const int wq_last = min(p.Nq - 1, q0 + kBlockRows - 1);
        wave_kend = max(0, min(p.Nk, wq_last + 1 + shift));
        wave_kmask = max(0, min(p.Nk, q0 + 1 + shift));  // keys below this are visible to all rows
    }
    if (q0 >= p.Nq) wave_kend = 0;  // padding block of a ragged last tile
    const int n_tiles = (wg_kend + kBN - 1) / kBN;

    // ---- Q fragments (B operand of S^T = K Q^T) ----
    const int qi = q0 + col;
    bf16x8 qf[KS];
    {
        const uint16_t* qp = p.q + ((size_t)(b * p.Hq + head) * p.Nq + (size_t)min(qi, p.Nq - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qi < p.Nq) x = *reinterpret_cast<const u32x4*>(qp + ks * 16 + half * 8);
            qf[ks] = as_bf16x8(x);
        }
    }
    // Causal limit of this lane's query (keys above it are masked).
    const int lim = CAUSAL ? min(p.Nk - 1, qi + shift) : p.Nk - 1;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float mref = -INFINITY;  // reference max, in exp2 units (score * scale_log2)
    float lsum = 0.0f;       // this lane half's share of the row sum

    const size_t kv_off = (size_t)(b * p.Hkv + g) * p.Nk * D;
    const uint16_t* kbase = p.k + kv_off;
    const uint16_t* vbase = p.v + kv_off;
    const int krow = key_of_row(col);  // K row this lane feeds to the MFMA

    if (n_tiles > 0) issue_tile<D>(kbase, vbase, smem, smem + Stage<D>::kBytesK, 0, p.Nk, wave, lane);

    for (int j = 0; j < n_tiles; ++j) {
        const int j0 = j * kBN;
        // Tile j's copies (this wave's) are done; the barrier publishes every
        // wave's copies and ends all reads of the other stage (tile j-1).
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (j + 1 < n_tiles) {
            lds_char* nst = smem + ((j + 1) & 1) * Stage<D>::kBytes;
            issue_tile<D>(kbase, vbase, nst, nst + Stage<D>::kBytesK, j0 + kBN, p.Nk, wave, lane);
        }
        if (j0 >= wave_kend) continue;  // wave-uniform: nothing visible for this block
        const lds_char* kst = smem + (j & 1) * Stage<D>::kBytes;
        const lds_char* vst = kst + Stage<D>::kBytesK;

        // ---- S^T = K Q^T for the two 32-key blocks (LDS reads two steps ahead) ----
        f32x16 s[kNKB];
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
        {
            u32x4 kf[KS][kNKB];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < kNKB; ++kb)
                    kf[ks][kb] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                        kst + tile_off<D>(kb * 32 + krow, 2 * ks + half));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < kNKB; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ks][kb]), qf[ks], s[kb], 0, 0, 0);
            // Keep the fragment reads two k-steps ahead of the MFMAs.
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kNKB, 0);
#pragma unroll
            for (int ks = 0; ks < KS - 2; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x008, kNKB, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, kNKB, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * kNKB, 0);
        }
        // ---- mask (only where some key of the tile is invisible to some row) ----
        if ((j0 + kBN > p.Nk) || (CAUSAL && j0 + kBN > wave_kmask)) {
#pragma unroll
            for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + kb * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                    if (key > lim) s[kb][r] = -INFINITY;
                }
        }
        // ---- online softmax ----
        float m = s[0][0];
#pragma unroll
        for (int i = 1; i + 1 < 16 * kNKB; i += 2)
            m = max3f(m, s[i >> 4][i & 15], s[(i + 1) >> 4][(i + 1) & 15]);
        m = fmaxf(m, s[kNKB - 1][15]);
        m = fmaxf(m, other_half(m));
        const float mx = m * p.scale_log2;
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
        const float ref = (mref == -INFINITY) ? 0.0f : mref;
        bf16x8 pf[2 * kNKB];
        float acc = 0.0f;
#pragma unroll
        for (int kb = 0; kb < kNKB; ++kb)
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                bf16x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][h8 * 8 + e], p.scale_log2, -ref));
                    acc += x;
                    pv[e] = (__bf16)x;
                }
                pf[kb * 2 + h8] = pv;
            }
        lsum += acc;
        // ---- O^T += V^T P^T (LDS reads two fragments ahead) ----
        {
            bf16x8 vf[2 * kNKB][DB];
#pragma unroll
            for (int t = 0; t < 2 * kNKB; ++t)
#pragma unroll
                for (int db = 0; db < DB; ++db) vf[t][db] = read_vt<D>(vst, db, t, lane);
#pragma unroll
            for (int t = 0; t < 2 * kNKB; ++t)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t][db], pf[t], oacc[db], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int i = 0; i < 2 * kNKB * DB - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        }
    }

    // ---- epilogue: O = O^T / l (transposed back on store), LSE = ln 2 * m + ln l ----
    const float l = lsum + other_half(lsum);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi < p.Nq) {
        const size_t row = (size_t)(b * p.Hq + head) * p.Nq + qi;
        uint16_t* op = p.o + row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dim = db * 32 + r4 * 8 + half * 4;
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                bf16x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[db][r4 * 4 + e] * inv);
                *reinterpret_cast<bf16x4*>(op + dim) = ov;
            }
        if (half == 0) p.lse[row] = l > 0.0f ? (mref * kLn2 + logf(l)) : -INFINITY;
    }
}

int pow2_divisor_upto8(int G) {
    int h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

template <int D, bool CAUSAL>
hipError_t launch_t(const FwdParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
    FwdParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.Nq = a.Nq; p.Nk = a.Nk;
    p.G = a.Hq / a.Hkv;
    p.heads_per_wg = pow2_divisor_upto8(p.G);
    p.qblocks_per_wg = kBlocksPerWG / p.heads_per_wg;
    p.n_hsub = p.G / p.heads_per_wg;
    const int rows_q = kBlockRows * p.qblocks_per_wg;
    p.n_qtiles = (a.Nq + rows_q - 1) / rows_q;
    p.n_units = a.B * a.Hkv * p.n_hsub;
    p.xcd_affine = (p.n_units % 8 == 0) ? 1 : 0;
    p.causal = a.causal;
    p.scale = a.scale;
    p.scale_log2 = a.scale * kLog2e;
    const long long grid = (long long)p.n_units * p.n_qtiles;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.d == 128) return a.causal ? launch_t<128, true>(p, (int)grid, stream) : launch_t<128, false>(p, (int)grid, stream);
    return a.causal ? launch_t<64, true>(p, (int)grid, stream) : launch_t<64, false>(p, (int)grid, stream);
}

}  // namespace fa
