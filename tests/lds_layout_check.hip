// Host-side check of the LDS tile layout helpers in fa_lds.h (the same
// functions the kernels call; they are pure integer functions). Exhaustive
// over rows, chunks, lanes and waves for both head dims. Prints one line per
// failed property and exits non-zero if any fails.
#include <cstdio>

#include "fa_lds.h"

using namespace fa::lds;

static int failures = 0;
#define CHECK(cond, ...)                      \
    do {                                      \
        if (!(cond)) {                        \
            if (failures < 20) {              \
                std::printf(__VA_ARGS__);     \
                std::printf("\n");            \
            }                                 \
            ++failures;                       \
        }                                     \
    } while (0)

template <int D>
static void check_dim() {
    constexpr int RB = D * 2;          // bytes per staged row
    constexpr int NC = RB / 16;        // 16-byte chunks per row
    constexpr int RPI = 1024 / RB;     // rows per 1 KiB copy block
    // The swizzle is a bijection on a row's chunks, and depends on the row
    // modulo 16 only (tiles are staged from rows that are multiples of 16).
    for (int r = 0; r < 256; ++r) {
        CHECK(swz<D>(r) >= 0 && swz<D>(r) < NC, "D=%d: swz(%d) = %d out of range", D, r, swz<D>(r));
        CHECK(swz<D>(r) == swz<D>(r % 16), "D=%d: swz(%d) depends on more than row mod 16", D, r);
        bool seen[NC] = {};
        for (int c = 0; c < NC; ++c) {
            const int o = tile_off<D>(r, c);
            const int slot = (o - r * RB) >> 4;
            CHECK(slot >= 0 && slot < NC && !seen[slot], "D=%d: row %d chunk %d maps to a taken slot", D, r, c);
            if (slot >= 0 && slot < NC) seen[slot] = true;
        }
    }
    // K fragment offsets of k-step ks (chunk 2 ks + h) from the k-step 0 base.
    for (int r = 0; r < 128; ++r)
        for (int h = 0; h < 2; ++h)
            for (int ks = 0; ks < D / 16; ++ks)
                CHECK(tile_off<D>(r, 2 * ks + h) == tile_off_ks(tile_off<D>(r, h), ks),
                      "D=%d: tile_off(%d, %d) != tile_off(%d, %d) ^ (%d << 5)", D, r, 2 * ks + h, r, h, ks);
    // Transposing-read offsets of dim block db from the block 0 base.
    for (int lane = 0; lane < 64; ++lane)
        for (int h = 0; h < 2; ++h)
            for (int db = 0; db < D / 32; ++db)
                CHECK(tr_off<D>(db, h, lane) == (tr_off<D>(0, h, lane) ^ (db << 6)),
                      "D=%d: tr_off(%d, %d, %d) is not the block 0 offset xor %d", D, db, h, lane, db << 6);
    // Scalar-base copies: a wave copies blocks blk = wave (mod W) of a tile
    // that starts at a row that is a multiple of 16; one lane offset must give
    // the same bytes as the per-lane form (row blk * RPI + lane / NC, chunk
    // (lane % NC) ^ swz(row)) for every such block.
    for (int W : {4, 8}) {
        for (int wave = 0; wave < W; ++wave)
            for (int lane = 0; lane < 64; ++lane) {
                const uint32_t voff = W == 4 ? stage_lane_offset<D, 4>(wave, lane) : stage_lane_offset<D, 8>(wave, lane);
                for (int blk = wave; blk * RPI < 256; blk += W) {
                    const int row = blk * RPI + lane / NC;
                    const int per_lane = row * RB + (((lane % NC) ^ swz<D>(row)) << 4);
                    CHECK((int)(blk * RPI * RB + voff) == per_lane,
                          "D=%d W=%d: wave %d lane %d block %d: lane offset %u != per-lane offset", D, W, wave, lane,
                          blk, voff);
                }
            }
    }
}

int main() {
    check_dim<64>();
    check_dim<128>();
    // The permuted K-row order fed to the MFMA is a bijection on 32 rows.
    bool seen[32] = {};
    for (int i = 0; i < 32; ++i) {
        const int r = row_of_mfma_row(i);
        CHECK(r >= 0 && r < 32 && !seen[r], "row_of_mfma_row(%d) = %d repeats or is out of range", i, r);
        if (r >= 0 && r < 32) seen[r] = true;
    }
    if (failures == 0) std::printf("lds layout: all properties hold\n");
    return failures == 0 ? 0 : 1;
}
