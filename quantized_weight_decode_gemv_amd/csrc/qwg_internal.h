// Internal interface between the C-ABI layer (qwg_api.cpp) and the kernel
// translation units (q4k.hip, iq3.hip). Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qwg {

constexpr int kQK = 256;
constexpr int kQ4kBytes = 144;
constexpr int kIq3Bytes = 98;
constexpr int kIq3sBytes = 110;   // IQ3_S (codebook formats)
constexpr int kIq4xsBytes = 136;  // IQ4_XS
// Format ids shared with the C ABI (QWG_FMT_* in qwg.h).
constexpr int kFmtIq3s = 3;
constexpr int kFmtIq4xs = 4;
constexpr int kTileRows = 64;  // one output row per lane of a wavefront

// One GEMV/GEMM problem as the kernels see it. `splits` workgroups share each
// 64-row tile, each summing a contiguous range of super-blocks; with
// splits > 1 they meet in `partial` ([splits][batch][tiles*64] fp32) and the
// last to arrive at `counters[tile]` adds the partial sums in split order.
struct GemvArgs {
    const uint8_t *w;
    const float *x;
    const float *grid;   // IQ3 only
    float *y;
    float *partial;
    uint32_t *counters;
    int64_t row_bytes;
    int n_in;
    int n_out;
    int nb;        // super-blocks per row
    int tiles;     // ceil(n_out / 64)
    int splits;    // 1..nb
    int wg_begin;  // first workgroup of this problem in a grouped launch
    int layout;    // kLayoutRows or kLayoutTiles (stream engine only)
};

// Weight layouts. Rows: row r is n_in/256 consecutive blocks, rows contiguous.
// Tiles (Q4_K): the same blocks ordered tile-major: for each 64-row tile, for
// each block column b, the 64 rows' block b back to back (9216 bytes); rows
// past n_out in the last tile are zero blocks. Block (r, b) sits at byte
// ((r/64)*nb + b)*9216 + (r%64)*144. Tiles (IQ3): the same column order, each
// 6272-byte column regrouped by field (described in iq3.hip). RowsXxs (IQ3
// only): row-major blocks in llama.cpp's IQ3_XXS byte order (d, indices, words)
// instead of the container's (indices, words, d).
constexpr int kLayoutRows = 0;
constexpr int kLayoutTiles = 1;
constexpr int kLayoutRowsXxs = 2;

// A grouped launch: problems[map[k]] is the problem of work item k (arrays in
// device memory). Without `tile`, the items of problem p are consecutive from
// problems[p].wg_begin and item k is tile k - wg_begin. With `tile` (the Q4_K
// stream engine's schedule), item k is tile tile[k] of problem map[k], and
// map[k] == kNoItem marks a position with no work.
struct GroupArgs {
    const GemvArgs *problems;
    const uint32_t *map;
    const uint32_t *tile;
};
constexpr uint32_t kNoItem = 0xFFFFFFFFu;

// Wavefronts per workgroup of the Q4_K GEMV (4, 8 or 16: one, two or four
// super-blocks of a 64-row tile per pipeline stage).
constexpr int kQ4kWavesSmall = 4;
constexpr int kQ4kWavesLarge = 16;

// Launchers: return hipSuccess or the launch error.
hipError_t launch_q4k_dequant(const uint8_t *src, float *dst, int64_t nblocks, hipStream_t s);
// Row-major Q4_K weights -> tile layout (dst: tiles*64*nb*144 bytes).
hipError_t launch_q4k_pack_tiles(const uint8_t *src, uint8_t *dst, int nb, int n_out, hipStream_t s);
// xxs: blocks in llama.cpp's IQ3_XXS byte order.
hipError_t launch_iq3_dequant(const uint8_t *src, const float *grid, float *dst,
                              int64_t nblocks, bool xxs, hipStream_t s);
hipError_t launch_q4k_gemv(const GemvArgs &a, int batch, int waves, hipStream_t s);
hipError_t launch_q4k_group(const GroupArgs &g, int total_workgroups, int max_nb, hipStream_t s);
// Batched GEMM on matrix cores (2 <= batch <= 8): one workgroup per (tile,
// split), `cols` super-block columns per stage (1: 4 wavefronts, ring of 2..4
// stages; 2: 8 wavefronts, ring of 2); `tiled`: weights in the Q4_K tile
// layout (ring of 2).
hipError_t launch_q4k_mfma(const GemvArgs &a, int batch, int ring, int cols, bool tiled,
                           hipStream_t s);
// The same engine over a group (g.problems with splits == 1, g.map item ->
// problem, problems[p].wg_begin its first item): `nwg` workgroups, one per
// 64-row tile of every member.
hipError_t launch_q4k_mfma_group(const GroupArgs &g, int nwg, int batch, int cols, bool tiled,
                                 hipStream_t s);
// Persistent stream engine (batch 1): `nitems` work items of the group
// (g.problems != nullptr) or of `single`; waves in {4, 8, 16}, ring stages in
// {2, 3}. split: some problem has splits > 1 (items are tile x range; each such
// problem carries its partial-sum workspace and zeroed tile counters).
hipError_t launch_q4k_stream(const GroupArgs &g, const GemvArgs &single, int nitems, int waves,
                             int ring, bool split, hipStream_t s);
// Resident workgroups per CU of that stream variant and the number of CUs
// (the launch grid is their product, capped by the item count); 0 if the
// variant does not exist.
int q4k_stream_residency(int waves, int ring, int *cus);
// Batched (2..8) persistent stream on the matrix cores: items of `single` (no
// group) or of a group's work list, an LDS ring of `ring` (2..4) stages across
// items; split: items may cover part of a row (partial sums meet through the
// problem's workspace).
int q4k_mstream_slots(int ring);
hipError_t launch_q4k_mstream(const GroupArgs &g, const GemvArgs &single, int nitems, int batch,
                              int ring, bool split, hipStream_t s);

// IQ3 stream engine shape: wavefronts per workgroup (4, 8, 16) and LDS ring
// stages (2, 3; 4 with 4 wavefronts).
struct Iq3Shape {
    int waves;
    int ring;
};
// Resident workgroups of that variant on the current device (0 if unsupported),
// for row-major or tile-layout weights.
int iq3_stream_slots(const Iq3Shape &sh, bool tiled);
// `nitems` work items (tile x split) of the group or of `single`; all members
// of a group share `grid` and the layout.
hipError_t launch_iq3_stream(const GroupArgs &g, const GemvArgs &single, const float *grid,
                             int nitems, const Iq3Shape &sh, bool tiled, hipStream_t s);
// Row-major IQ3 weights (container or, with xxs, llama.cpp order) -> tile
// layout (dst: tiles*64*nb*98 bytes; the same layout for both orders).
hipError_t launch_iq3_pack_tiles(const uint8_t *src, uint8_t *dst, int nb, int n_out, bool xxs,
                                 hipStream_t s);

// Codebook formats IQ3_S / IQ4_XS (codebook.hip). Dequant: bit-exact. GEMV:
// persistent 4-wavefront workgroups on the tile layout (launch_cb_pack_tiles
// makes it) or on row-major blocks; `tab` is the [512][4] grid (IQ3_S) or the
// 16-value table (IQ4_XS).
hipError_t launch_iq3s_dequant(const uint8_t *src, const float *grid, float *dst, int64_t nblocks,
                               hipStream_t s);
hipError_t launch_iq4xs_dequant(const uint8_t *src, const float *table, float *dst,
                                int64_t nblocks, hipStream_t s);
hipError_t launch_cb_pack_tiles(int fmt, const uint8_t *src, uint8_t *dst, int nb, int n_out,
                                hipStream_t s);
// Engine shape (10 * wavefronts + ring stages; wavefronts / 4 super-blocks per
// pipeline stage) of a launch that splits its sums (split) or not.
int cb_stream_shape(int fmt, bool split);
// resident workgroups of the tile-layout (tiled) or row-major engine of that
// shape on the current device (0: unknown format or shape)
int cb_stream_slots(int fmt, bool tiled, int shape);
// tiled: the tile layout; otherwise row-major blocks, w 16-byte aligned
// Row-group kernel for IQ3_S / IQ4_XS single GEMVs (a.layout rows or tiles,
// rows of nb <= 24 blocks): eight whole rows per workgroup, no split sums.
bool cb_rows_fits(int nb);
hipError_t launch_cb_rows(int fmt, const GemvArgs &a, const float *tab, hipStream_t s);
hipError_t launch_cb_stream(int fmt, bool tiled, int shape, const GroupArgs &g,
                            const GemvArgs &single, const float *tab, int nitems, hipStream_t s);

// Layer-chain launch (chain.hip): a decoder's Q4_K weight stream in phases that
// run in dependency order inside one persistent launch (tile-layout weights).
// One workgroup of kChainQuads x 4 wavefronts per compute unit; each quad
// computes at most one unit per phase: one 64-row tile of one member over
// nblk <= kChainMaxSteps consecutive super-block columns.
constexpr int kChainQuads = 4;
constexpr int kChainRing = 4;      // LDS ring slots (columns per quad)
constexpr int kChainMaxSteps = 2;  // columns per unit
constexpr int kFlagCopies = 8;     // one copy of the flags per XCD
constexpr int kFlagCopyWords = 1024;   // 4 KB apart
// How a member's rows are completed: a unit covers whole rows (direct); units
// store partial sums that the launch adds up at its end (deferred); or, for a
// member whose y a later phase reads, the tile's last unit adds them up at
// once (wired).
constexpr int kChainDirect = 0;
constexpr int kChainDeferred = 1;
constexpr int kChainWired = 2;

struct ChainMember {
    const uint8_t *w;     // tile layout
    const float *x;
    float *y;
    float *partial;       // [splits][tiles*64] fp32 (splits > 1)
    uint32_t *counters;   // [tiles] (wired members)
    // Tagged launches: a member whose y a later member reads publishes each
    // row (each row's partial sum per split) as a tagged pair, fp32 bits | tag
    // << 32, in `ll` [splits][n_out]; a member that reads such a y finds
    // activation k of split s at xll[s * xstride + k], sums the xsplits
    // partials in split order and waits for the tags. A member of any phase
    // but the last marks each finished (tile, split) with a tagged done word.
    uint64_t *ll;         // [splits][n_out] (producers), else null
    const uint64_t *xll;  // the producer's ll at this member's x (consumers), else null
    uint64_t *done;       // [tiles][splits], else null
    int xsplits;          // consumers: the producer's splits
    int xstride;          // consumers: the producer's n_out
    int n_out;
    int nb;
    int tiles;
    int splits;           // units per tile
    int mode;
    int tag;              // producers: the tag written is run base + tag
    int xtag;             // consumers: the producer's tag
    int pad;
};

// units: [nphases][nwg*kChainQuads] entries of four uint32 (member or kNoItem,
// tile, b0 | nblk << 8 | split << 16, 0); phases: [nphases] entries of four
// uint32 (columns of the phase; barrier launches: 1 if it waits for the
// previous phase, tagged launches: the tag offset of the done words it waits
// for; how many done words; their first index in `done`); fin: [nfin] pairs
// (member, tile) of the deferred members' tiles; flags: one per workgroup
// (phases completed, counted across runs), kFlagCopies copies kFlagCopyWords
// apart; err: set when a wait gave up. tagged: a phase waits for the done
// words of the previous phase's tiles and reads activations produced in the
// chain as tagged rows, instead of a flag barrier over every workgroup.
struct ChainArgs {
    const ChainMember *members;
    const uint32_t *units;
    const uint32_t *phases;
    const uint32_t *fin;
    const uint64_t *done;
    uint32_t *flags;
    uint32_t *err;
    int nphases;
    int nfin;
    int nwg;
    int tagged;
};
hipError_t launch_q4k_chain(const ChainArgs &c, hipStream_t s);
int chain_lds_bytes();

// IQ3 container encoder (encode.hip): x [nblocks][256] fp32 -> nblocks 98-byte
// blocks, grid [256][4] in weight units.
hipError_t launch_iq3_encode(const float *x, const float *grid, uint8_t *dst, int64_t nblocks,
                             hipStream_t s);

}  // namespace qwg
