// Interface of the short-call GEMV kernel (short.hip): a single GEMV of a few
// MB spread over up to one workgroup per compute unit, each requesting every
// byte it needs in its first instructions, so that one memory round trip later
// the dot products run. Not installed.
#pragma once

#include "qwg_internal.h"

namespace qwg {

// A workgroup holds at most this many Q4_K super-block columns of one 64-row
// tile, one per four wavefronts.
constexpr int kShortMaxBlocks = 4;
// Splits of a tile's super-block range, and tiles, that a short call supports:
// the grid (tiles x splits) is at most one workgroup per compute unit, so every
// workgroup of a launch is resident at once on an otherwise idle device.
constexpr int kShortMaxSplits = 8;
constexpr int kShortMaxTiles = 256;
// Split words: [tile][split][64 rows] 8-byte tagged partial sums, then one
// 32-bit epoch per tile (zeroed when the workspace is created).
constexpr size_t kShortWords = (size_t)kShortMaxTiles * kShortMaxSplits * kTileRows;
constexpr size_t kShortEpochs = kShortMaxTiles;

// Launch grid of a short call: position b runs on XCD b % 8, and the splits of
// tile t share XCD t % 8 (b = 8 (S (t / 8) + split) + t % 8), so that a split
// tile's neighbouring block columns (row-major blocks share cache lines) and
// its tagged words meet in one L2. Positions past the last tile are idle.
// Measured against tile-major order (same box, alternating runs): 2048 x
// 2048 5.16 -> 4.80 us, 256 x 2048 4.60 -> 4.08, 2048 x 5632 6.40 -> 6.08.
inline int short_grid(int tiles, int splits) { return 8 * splits * ((tiles + 7) / 8); }

struct ShortState {
    uint64_t *words;   // kShortWords
    uint32_t *epochs;  // kShortEpochs
};

// Splits for a Q4_K or IQ3 short call of `tiles` tiles and `nb` super-blocks per row
// on `cus` compute units (as many as fit: tiles x splits <= cus, splits <=
// min(nb, kShortMaxSplits)), or 0 if the call does not qualify (more tiles
// than compute units, or more than kShortMaxBlocks columns per workgroup).
int short_plan_splits(int tiles, int nb, int cus);
// a.splits set by the caller (short_plan_splits); st needed when a.splits > 1.
hipError_t launch_q4k_short(const GemvArgs &a, const ShortState &st, bool tiled, hipStream_t s);
// Row-group kernel (Q4_K, batch 1, rows of nb <= 8 super-blocks): eight whole
// rows per workgroup, no split sums (so no workspace).
bool q4k_rows_fits(int nb);
hipError_t launch_q4k_rows(const GemvArgs &a, bool tiled, hipStream_t s);
// Row-group kernel for IQ3 (any layout, rows of nb <= 24 blocks), the same scheme.
// Bytes per block of the IQ3 tile layout (qwg_pack_iq3_tiles): the 98-byte
// block's fields regrouped, with the sign bit that each group's even-count
// rule implies written out (32 more bits per block).
constexpr int kIq3TileBlock = 102;
bool iq3_rows_fits(int nb);
hipError_t launch_iq3_rows(const GemvArgs &a, const float *grid, hipStream_t s);
// IQ3 (a.layout: rows, llama.cpp-order rows or tiles), the same plan rule.
hipError_t launch_iq3_short(const GemvArgs &a, const ShortState &st, const float *grid,
                            hipStream_t s);

}  // namespace qwg
