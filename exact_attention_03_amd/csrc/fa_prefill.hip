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
//   * Workgroup = 4 waves = 8 row blocks of 32 queries. A row block is 32
//     consecutive queries of one query head. The 8 blocks of a workgroup
//     share one K/V head (GQA packing): for a group size G they are
//     min(G, 8) heads x (8 / min(G, 8)) query blocks. Wave w owns blocks w
//     and w + 4, i.e. 64 rows.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 result each lane holds one query
//     (column) and 16 keys (rows), so the softmax max / sum are in-lane
//     reductions plus one exchange between the two 32-lane halves.
//   * The K rows fed to the MFMA are permuted so that result register r of
//     lane half h holds key 16*(r/8) + 8*h + r%8 of the 32-key block. The
//     exponentiated scores then already form the B operand of the second MFMA,
//     O^T += V^T P^T, with keys in natural order -- no data movement.
//   * K is staged row-major and V transposed (V^T) in LDS, both with an XOR
//     swizzle of 16-byte chunks so that the MFMA operand reads are free of
//     bank conflicts; two LDS stages let the loads of tile j+1 overlap the
//     math of tile j.
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

constexpr int kThreads = 256;
constexpr int kBN = 64;             // keys per K/V tile
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

// Byte offset of 16-byte chunk `c` of row `r` in the K stage (row-major,
// D/8 chunks per row, XOR-swizzled).
template <int D>
__device__ __forceinline__ int k_lds_off(int r, int c) {
    if constexpr (D == 128) return r * 256 + ((c ^ (r & 15)) << 4);
    else return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
// Byte offset of 16-byte chunk `c` (8 keys) of dim-row `r` in the V^T stage
// (D rows of 64 keys = 128 bytes, XOR-swizzled).
__device__ __forceinline__ int vt_lds_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Key held by MFMA row index i of a 32-key block (see the file header).
__device__ __forceinline__ int key_of_row(int i) {
    int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
    return ((a >> 1) << 4) + (h << 3) + ((a & 1) << 2) + b;
}

template <int D>
struct Stage {
    static constexpr int kBytesK = kBN * D * 2;
    static constexpr int kBytesV = kBN * D * 2;
    static constexpr int kBytes = kBytesK + kBytesV;
    static constexpr int kLoadsK = kBN * D / 8 / kThreads;  // 16-byte K chunks per thread
    static constexpr int kKPT = D / 32;                     // V keys per thread
};

// Registers holding one K/V tile on its way from global memory to LDS.
template <int D>
struct TileRegs {
    u32x4 k[Stage<D>::kLoadsK];
    u32x4 v[Stage<D>::kKPT];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int j0, int Nk, int tid) {
    constexpr int CH = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < Stage<D>::kLoadsK; ++i) {
        int r = tid / CH + (kThreads / CH) * i;
        int c = tid % CH;
        int key = j0 + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < Nk) x = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D + c * 8);
        t.k[i] = x;
    }
    constexpr int KPT = Stage<D>::kKPT;
    constexpr int NKG = kBN / KPT;  // key groups
    int kg = tid % NKG, cg = tid / NKG;
#pragma unroll
    for (int kk = 0; kk < KPT; ++kk) {
        int key = j0 + kg * KPT + kk;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < Nk) x = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * D + cg * 8);
        t.v[kk] = x;
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, char* __restrict__ kst,
                                           char* __restrict__ vst, int tid) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int i = 0; i < Stage<D>::kLoadsK; ++i) {
        int r = tid / CH + (kThreads / CH) * i;
        int c = tid % CH;
        *reinterpret_cast<u32x4*>(kst + k_lds_off<D>(r, c)) = t.k[i];
    }
    constexpr int KPT = Stage<D>::kKPT;
    constexpr int NKG = kBN / KPT;
    int kg = tid % NKG, cg = tid / NKG;
    int key0 = kg * KPT;
    int chunk = key0 >> 3, inb = (key0 & 7) * 2;
#pragma unroll
    for (int w = 0; w < 4; ++w) {        // dword w of each loaded chunk = dims 2w, 2w+1
#pragma unroll
        for (int s = 0; s < 2; ++s) {    // s = 0: even dim, 1: odd dim
            const uint32_t sel = s ? 0x07060302u : 0x05040100u;
            int row = cg * 8 + 2 * w + s;
            char* dst = vst + vt_lds_off(row, chunk) + inb;
            if constexpr (KPT == 4) {
                u32x2 pr;
                pr.x = __builtin_amdgcn_perm(t.v[1][w], t.v[0][w], sel);
                pr.y = __builtin_amdgcn_perm(t.v[3][w], t.v[2][w], sel);
                *reinterpret_cast<u32x2*>(dst) = pr;
            } else {
                *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(t.v[1][w], t.v[0][w], sel);
            }
        }
    }
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Value of x in lane l^32 (the other 32-lane half).
__device__ __forceinline__ float other_half(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    int lane = __lane_id();
    return __uint_as_float(lane < 32 ? s[1] : s[0]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_fwd_kernel(FwdParams p) {
    constexpr int KS = D / 16;   // 16-dim k-steps of Q K^T
    constexpr int DB = D / 32;   // 32-dim blocks of O^T
    extern __shared__ __attribute__((aligned(16))) char smem[];

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

    // ---- this wave's two row blocks ----
    int head[2], q0[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int blk = wave + 4 * i;
        const int hi = blk / p.qblocks_per_wg, qb = blk % p.qblocks_per_wg;
        head[i] = g * p.G + hsub * p.heads_per_wg + hi;
        q0[i] = qtile0 + qb * kBlockRows;
    }
    const int shift = p.Nk - p.Nq;  // causal: key j visible from query i iff j <= i + shift

    // Key range of the workgroup and of this wave.
    int wg_kend = p.Nk, wave_kend = p.Nk, wave_kmask = p.Nk;
    if (CAUSAL) {
        const int wg_qlast = min(p.Nq, qtile0 + rows_q) - 1;
        wg_kend = max(0, min(p.Nk, wg_qlast + 1 + shift));
        const int wq_last = min(p.Nq - 1, max(q0[0], q0[1]) + kBlockRows - 1);
        wave_kend = max(0, min(p.Nk, wq_last + 1 + shift));
        const int wq_first = min(q0[0], q0[1]);
        wave_kmask = max(0, min(p.Nk, wq_first + 1 + shift));  // keys below this are visible to all rows
    }
    const int n_tiles = (wg_kend + kBN - 1) / kBN;

    // ---- Q fragments (B operand of S^T = K Q^T) ----
    bf16x8 qf[2][KS];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int qi = q0[i] + col;
        const uint16_t* qp = p.q + ((size_t)(b * p.Hq + head[i]) * p.Nq + (size_t)min(qi, p.Nq - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qi < p.Nq) x = *reinterpret_cast<const u32x4*>(qp + ks * 16 + half * 8);
            qf[i][ks] = as_bf16x8(x);
        }
    }

    f32x16 oacc[2][DB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][db][r] = 0.0f;
    float mref[2] = {-INFINITY, -INFINITY};  // reference max, in exp2 units (score * scale_log2)
    float lsum[2] = {0.0f, 0.0f};            // this lane half's share of the row sum

    const size_t kv_off = (size_t)(b * p.Hkv + g) * p.Nk * D;
    const uint16_t* kbase = p.k + kv_off;
    const uint16_t* vbase = p.v + kv_off;
    const int krow = key_of_row(col);  // K row this lane feeds to the MFMA

    TileRegs<D> tr;
    if (n_tiles > 0) {
        load_tile<D>(tr, kbase, vbase, 0, p.Nk, tid);
        store_tile<D>(tr, smem, smem + Stage<D>::kBytesK, tid);
    }
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int j0 = j * kBN;
        if (j + 1 < n_tiles) load_tile<D>(tr, kbase, vbase, j0 + kBN, p.Nk, tid);
        const char* kst = smem + (j & 1) * Stage<D>::kBytes;
        const char* vst = kst + Stage<D>::kBytesK;

        if (j0 < wave_kend) {
            // ---- S^T = K Q^T for the two 32-key blocks and the two row blocks ----
            f32x16 s[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[i][kb][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        kst + k_lds_off<D>(kb * 32 + krow, 2 * ks + half)));
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        s[i][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i][ks], s[i][kb], 0, 0, 0);
                }
            }
            // ---- mask (only where some key of the tile is invisible to some row) ----
            const bool need_mask = (j0 + kBN > p.Nk) || (CAUSAL && j0 + kBN > wave_kmask);
            if (need_mask) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int lim = CAUSAL ? min(p.Nk - 1, q0[i] + col + shift) : p.Nk - 1;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = j0 + kb * 32 + ((r >> 3) << 4) + (half << 3) + (r & 7);
                            if (key > lim) s[i][kb][r] = -INFINITY;
                        }
                }
            }
            // ---- online softmax ----
            float mx[2];
            bool grow = false;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float m = s[i][0][0];
#pragma unroll
                for (int r = 1; r < 15; r += 2) m = max3f(m, s[i][0][r], s[i][0][r + 1]);
                m = max3f(m, s[i][0][15], s[i][1][0]);
#pragma unroll
                for (int r = 1; r < 15; r += 2) m = max3f(m, s[i][1][r], s[i][1][r + 1]);
                m = fmaxf(m, s[i][1][15]);
                m = fmaxf(m, other_half(m));
                mx[i] = m * p.scale_log2;
                grow |= mx[i] > mref[i] + kRescaleSlack;
            }
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float mnew = fmaxf(mref[i], mx[i]);
                    const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mref[i] - mnew);
                    mref[i] = mnew;
                    lsum[i] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[i][db][r] *= alpha;
                }
            }
            bf16x8 pf[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float ref = (mref[i] == -INFINITY) ? 0.0f : mref[i];
                float acc = 0.0f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h8 = 0; h8 < 2; ++h8) {
                        bf16x8 pv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i][kb][h8 * 8 + e], p.scale_log2, -ref));
                            acc += x;
                            pv[e] = (__bf16)x;
                        }
                        pf[i][kb * 2 + h8] = pv;
                    }
                lsum[i] += acc;
            }
            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        vst + vt_lds_off(db * 32 + col, 2 * t + half)));
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        oacc[i][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[i][t], oacc[i][db], 0, 0, 0);
                }
            }
        }
        if (j + 1 < n_tiles) {
            char* nst = smem + ((j + 1) & 1) * Stage<D>::kBytes;
            store_tile<D>(tr, nst, nst + Stage<D>::kBytesK, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l (transposed back on store), LSE = ln 2 * m + ln l ----
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int qi = q0[i] + col;
        const float l = lsum[i] + other_half(lsum[i]);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        if (qi < p.Nq) {
            const size_t row = (size_t)(b * p.Hq + head[i]) * p.Nq + qi;
            uint16_t* op = p.o + row * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int dim = db * 32 + r4 * 8 + half * 4;
                    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                    bf16x4 ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[i][db][r4 * 4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(op + dim) = ov;
                }
            if (half == 0) p.lse[row] = l > 0.0f ? (mref[i] * kLn2 + logf(l)) : -INFINITY;
        }
    }
}

int pow2_divisor_upto8(int G) {
    int h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

template <int D, bool CAUSAL>
hipError_t launch_t(const FwdParams& p, int grid, hipStream_t stream) {
    const size_t smem = 2 * Stage<D>::kBytes;
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), smem, stream, p);
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
