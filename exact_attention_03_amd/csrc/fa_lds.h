// LDS tile and lane helpers shared by the gfx950 attention kernels (bf16
// forward, FP8 forward, backward).
//
// A staged tile is `rows` rows of D bf16 values, row-major, each row's
// 16-byte chunks XOR-swizzled by a function of the row so that both the
// 16-byte operand reads of 16 consecutive rows at one chunk and the
// transposing reads (ds_read_b64_tr_b16) of 4 rows x 4 chunks are free of
// bank conflicts. Rows are copied global -> LDS with global_load_lds_dwordx4
// (1 KiB per wave instruction).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace lds {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// XOR swizzle of the 16-byte chunks of a staged bf16 row: a bijection on the
// row's chunks; for 16 consecutive rows read at one chunk (operand reads)
// and for 4 consecutive rows x 4 consecutive chunks (transposing reads)
// every 16-lane phase lands on distinct bank groups.
template <int D>
__host__ __device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of logical 16-byte chunk c of row r in a staged tile.
template <int D>
__host__ __device__ __forceinline__ int tile_off(int r, int c) { return r * (D * 2) + ((c ^ swz<D>(r)) << 4); }

// Row of a 32-row block that MFMA row index i (0..31) reads, chosen so that
// result register r of lane half h of v_mfma_f32_32x32x16 holds row
// 16*(r/8) + 8*h + r%8: the 16 results of a lane are then 8 consecutive
// rows of each 16-row slice, i.e. already the B operand of a second MFMA
// whose reduction runs over those rows.
__host__ __device__ __forceinline__ int row_of_mfma_row(int i) {
    int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
    return ((a >> 1) << 4) + (h << 3) + ((a & 1) << 2) + b;
}

// 16 bytes per lane from global memory to LDS at lds_base + 16 * lane.
// lds_base is wave-uniform and goes through M0 (one wait state before the
// copy reads it). Issued from asm so the compiler does not make later reads
// of other LDS stages wait for it; callers wait (s_waitcnt vmcnt) before the
// barrier that publishes the stage.
__device__ __forceinline__ void copy16_to_lds(const void* gptr, uint32_t lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(base) : "memory", "m0");
}

// Copy rows [r0, r0 + ROWS) of a row-major [n_rows, D] bf16 matrix into a
// staged tile, with WAVES waves sharing the work. Rows at or past n_rows are
// clamped to the last row (n_rows >= 1): callers mask them.
template <int D, int ROWS, int WAVES>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ base, lds_char* st, int r0, int n_rows,
                                           int wave, int lane) {
    constexpr int RB = D * 2;       // bytes per row
    constexpr int RPI = 1024 / RB;  // rows per wave instruction
    constexpr int NI = ROWS * RB / 1024 / WAVES;
    static_assert(NI >= 1 && NI * WAVES * 1024 == ROWS * RB, "tile must split into whole 1 KiB wave copies");
    const int uw = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int blk = n * WAVES + uw;
        const int r = blk * RPI + lane / (RB / 16);
        const int c = (lane % (RB / 16)) ^ swz<D>(r);
        const int row = min(r0 + r, n_rows - 1);
        copy16_to_lds(base + (size_t)row * D + c * 8, (uint32_t)(uintptr_t)(st + blk * 1024));
    }
}

// 4 bytes per lane from global memory to LDS at lds_base + 4 * lane
// (global_load_lds_dword), under the same rules as copy16_to_lds().
__device__ __forceinline__ void copy4_to_lds(const void* gptr, uint32_t lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(gptr), "s"(base) : "memory", "m0");
}

// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (the saddr form): no per-lane address arithmetic.
__device__ __forceinline__ void copy16_to_lds_sbase(uint32_t voff, const uint16_t* sbase, uint32_t lds_base) {
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lb)
                 : "memory", "m0");
}

// Per-lane byte offset, within the RPI rows one wave instruction copies, of
// this lane's 16 bytes for stage_rows_full(). With r0 a multiple of 16, a
// wave's copies start at rows congruent to wave * RPI modulo 16, and the
// swizzle only depends on the row modulo 16: one offset serves them all.
template <int D, int WAVES>
__host__ __device__ __forceinline__ uint32_t stage_lane_offset(int wave, int lane) {
    constexpr int RB = D * 2;
    constexpr int RPI = 1024 / RB;
    static_assert((WAVES * RPI) % 16 == 0, "a wave's copy rows must keep their residue mod 16");
    const int rl = lane / (RB / 16);
    const int c = (lane % (RB / 16)) ^ swz<D>((wave % WAVES) * RPI + rl);
    return (uint32_t)(rl * RB + c * 16);
}

// stage_rows() for a tile that lies wholly below n_rows, with r0 a multiple
// of 16: scalar bases and the lane offset voff = stage_lane_offset().
template <int D, int ROWS, int WAVES>
__device__ __forceinline__ void stage_rows_full(const uint16_t* __restrict__ base, lds_char* st, int r0, uint32_t voff,
                                                int wave) {
    constexpr int RB = D * 2;
    constexpr int RPI = 1024 / RB;
    constexpr int NI = ROWS * RB / 1024 / WAVES;
    static_assert(NI >= 1 && NI * WAVES * 1024 == ROWS * RB, "tile must split into whole 1 KiB wave copies");
    const int uw = __builtin_amdgcn_readfirstlane(wave % WAVES);
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int blk = n * WAVES + uw;
        copy16_to_lds_sbase(voff, base + (size_t)(r0 + blk * RPI) * D, (uint32_t)(uintptr_t)(st + blk * 1024));
    }
}

// Byte offsets of this lane's two transposing reads for dim block db of
// 16-row slice 0 of a staged tile: A operand of (D x rows) x (rows x 32)
// products, dims 32*db + lane%32, rows 8*(lane/32) .. +7. Slice t adds 16*t
// rows (the swizzle only depends on the row modulo 16).
template <int D>
__host__ __device__ __forceinline__ int tr_off(int db, int h, int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int dim = db * 32 + 16 * (G & 1) + 4 * (j & 3);
    const int row = 8 * (G >> 1) + (j >> 2) + 4 * h;
    return tile_off<D>(row, dim >> 3) + (dim & 7) * 2;
}

// The swizzle only touches the low bits of a chunk index that the k-step
// and dim-block terms leave alone, so offsets differ from block 0 by an xor:
//   tile_off(r, 2 ks + h) == tile_off(r, h) ^ (ks << 5)
//   tr_off(db, h, lane)   == tr_off(0, h, lane) ^ (db << 6)
// (D = 64 and 128, every row, lane and half; checked exhaustively).
__host__ __device__ __forceinline__ int tile_off_ks(int off0, int ks) { return off0 ^ (ks << 5); }

// read_tr() from the block-0 offsets off0[h] = tr_off(0, h, lane).
template <int D>
__device__ __forceinline__ bf16x8 read_tr_db(const lds_char* st, const int (&off0)[2], int db, int t) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + (off0[0] ^ (db << 6)) + t * 16 * (D * 2)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + (off0[1] ^ (db << 6)) + t * 16 * (D * 2)));
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

template <int D>
__device__ __forceinline__ bf16x8 read_tr(const lds_char* st, const int (&off)[D / 32][2], int db, int t) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + off[db][0] + t * 16 * (D * 2)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + off[db][1] + t * 16 * (D * 2)));
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// 16-byte operand read of chunk c of row r of a staged tile.
template <int D>
__device__ __forceinline__ bf16x8 read_row(const lds_char* st, int r, int c) {
    return as_bf16x8(*reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(st + tile_off<D>(r, c)));
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Value of x in lane l ^ 32 (the other 32-lane half).
__device__ __forceinline__ float other_half(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(__lane_id() < 32 ? s[1] : s[0]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace lds
}  // namespace fa
