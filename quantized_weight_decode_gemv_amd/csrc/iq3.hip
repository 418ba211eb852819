// IQ3 ("fmt=5" grouped container) kernels for gfx950: dequantization and GEMV.
//
// Format: iq3_pack.py page, module docstring and decode(). A 98-byte block of
// 256 weights holds 64 grid indices (bytes 0-63, index 8ib + t/4 for weight t of
// sub-block ib), eight little-endian uint32 words (64-95, one per 32-weight
// sub-block: bits 7l..7l+6 are the signs of weights 8l..8l+6, the sign of weight
// 8l+7 is their XOR, bits 28-31 the sub-scale code) and fp16 d (96-97).
// Weight = grid[idx][t%4] * sign * db, db = d*(0.5+code)*0.5; every factor has
// few enough significant bits that the fp32 product is exact.
//
// GEMV: a persistent stream engine (described above iq3_stream below) with the
// grid expanded once per workgroup into a sign-folded table in LDS, so that four
// weights cost one v_perm, one LDS read and four FMAs; the eighth sign of each
// 8-weight group is rebuilt for all four groups of a word at once with
// byte-parallel XOR folding.
#include "qwg_device.h"
#include "short_dev.h"

namespace qwg {

namespace {

__device__ __forceinline__ uint32_t load_u16(const uint8_t *p) {
    return *(const uint16_t *)p;
}

// Little-endian 32-bit word at a 2-byte aligned address.
__device__ __forceinline__ uint32_t load_u32_a2(const uint8_t *p) {
    return load_u16(p) | (load_u16(p + 2) << 16);
}

// Four 7-bit sign groups (word bits 0-27) -> one byte per group with the parity
// bit in bit 7, i.e. bit t of the result is the sign of weight t (1 = negative).
__device__ __forceinline__ uint32_t iq3_signs(uint32_t word) {
    const uint32_t t = (word & 0x3FFFu) | ((word << 2) & 0x3FFF0000u);
    const uint32_t u = (t & 0x007F007Fu) | ((t << 1) & 0x7F007F00u);
    uint32_t p = u ^ (u >> 4);
    p ^= p >> 2;
    p ^= p >> 1;
    return u | ((p & 0x01010101u) << 7);
}

// Field offsets of a 98-byte block in the two byte orders: the iq3_pack
// container (indices at 0, words at 64, d at 96) and llama.cpp's IQ3_XXS
// (d at 0, indices at 2, words at 66), which the codebook.py page's format
// table describes. The fields and the decode are the same.
struct Iq3Order {
    int idx, words, d;
};
__device__ __forceinline__ Iq3Order iq3_order(bool xxs) {
    return xxs ? Iq3Order{2, 66, 0} : Iq3Order{0, 64, 96};
}

// ------------------------------------------------------------------ dequant

// One wavefront per block: lane l produces weights 4l..4l+3, i.e. the four
// magnitudes of grid row idx[l] of sub-block l/8.
__global__ __launch_bounds__(256) void iq3_dequant_kernel(const uint8_t *__restrict__ src,
                                                          const float *__restrict__ grid,
                                                          float *__restrict__ dst,
                                                          int64_t nblocks, bool xxs) {
    const Iq3Order fo = iq3_order(xxs);
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int ib = lane >> 3;         // sub-block
    const int t0 = 4 * (lane & 7);    // first weight of this lane within the sub-block
    for (int64_t blk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
         blk < nblocks; blk += nwaves) {
        const uint8_t *b = src + blk * kIq3Bytes;
        const float d = h2f_lo(load_u16(b + fo.d));
        const uint32_t word = load_u32_a2(b + fo.words + 4 * ib);
        const uint32_t code = word >> 28;
        const float db = __fmul_rn(__fmul_rn(d, 0.5f + (float)code), 0.5f);
        const uint32_t s8 = iq3_signs(word);
        const float4 g = *(const float4 *)(grid + 4 * b[fo.idx + lane]);
        float4 o;
        o.x = __fmul_rn(((s8 >> (t0 + 0)) & 1u) ? -g.x : g.x, db);
        o.y = __fmul_rn(((s8 >> (t0 + 1)) & 1u) ? -g.y : g.y, db);
        o.z = __fmul_rn(((s8 >> (t0 + 2)) & 1u) ? -g.z : g.z, db);
        o.w = __fmul_rn(((s8 >> (t0 + 3)) & 1u) ? -g.w : g.w, db);
        // written once: non-temporal, as the Q4_K dequant's stores
        __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, (f32x4 *)(dst + blk * kQK + 4 * lane));
    }
}

// ------------------------------------------------------------------ GEMV
//
// Persistent stream engine: a grid of about one workgroup per resident slot of
// the chip walks work items k, k + grid, ...; an item is one 64-row tile of one
// matrix over a contiguous range of super-blocks (the whole row, or one of
// `splits` ranges whose partial sums meet in tile_epilogue). Wavefront 4j + G
// computes sub-blocks 2G and 2G+1 of the j-th super-block of every pipeline
// stage for all 64 rows (lane r = row r of the tile), so its 64 activations
// are wave-uniform and come through scalar loads. An R-slot LDS ring, filled by
// LDS-DMA, runs ahead across item boundaries.
//
// Staging: a 98-byte block starts at any even address, so each row's block is
// copied as the seven naturally aligned 16-byte granules that cover it (a
// 112-byte window: 14 + 98 <= 7*16) and lanes re-align with v_alignbyte. Every
// granule address is clamped into the granules lying wholly inside the weight
// buffer, so nothing outside it is read. Only two granules can be affected:
// the first one of a buffer that starts off a 16-byte boundary (row 0's first
// block) and the last one of a buffer that ends off one (the last row's last
// block); the lane of that row takes that block's bytes from direct 2-byte
// loads instead.
//
// Grid: the workgroup stages the [256][4] fp32 grid in LDS once and expands it
// into a sign-folded fp16 table T[s][i] = (+-g_i0, +-g_i1, +-g_i2, +-g_i3) for
// the 16 sign patterns s of a group of four weights (bit c of s negates
// component c), entry (s, i) at LDS byte s*2048 + i*8 (32 KB), so four weights
// cost one v_perm (s*256 + i from the sign nibble and the index byte), one
// shift, one 8-byte LDS read and four FMAs. fp16 holds the magnitudes exactly
// when they are fp16 values (the small integers IQ3 grids use). A 64 KB layout
// with the address straight out of the v_perm (entry at i*256 + s*16) measured
// slower: its bank depends on s alone, so lanes collide far more often.
// Tile layout (qwg_pack_iq3_tiles): for each 64-row tile and block column b,
// 6528 bytes = the 64 rows' blocks regrouped by field and wavefront role, with
// the signs written out: index bytes [G][row][16] (bytes 16G..16G+15 of each
// block, 4 x 1024 B); sign bytes [G][row][8] (sub-blocks 2G and 2G+1, four
// bytes each: byte k holds group k's seven stored signs and, in bit 7, the
// eighth, the one the even-count rule implies; 4 x 512 B); sub-block scales
// [G][row] (scale of sub-block 2G in the low nibble, 2G+1 in the high one;
// 4 x 64 B); then d [row][2] (128 B). 102 bytes per block against the
// container's 98: the 32 implied signs are stored, so the dot takes each sign
// nibble with one mask instead of the ~11 VALU ops per word that recover the
// eighth sign and move the 7-bit groups apart (measured on the grouped IQ3
// stream, a copy of the kernel that skipped that step: 90.6 -> 81.6 us).
// Column (t, b) starts at (t*nb + b) * 6528; rows past n_out are zero blocks.
// A stage copy is contiguous, and wavefront G's lanes (rows) read consecutive
// 16-, 8-, 1- and 2-byte pieces: no realignment, no bank conflicts, no clamping.
constexpr int kIq3TileSigns = 4096;
constexpr int kIq3TileScales = 6144;
constexpr int kIq3TileD = 6400;
constexpr int kIq3TileCol = 6528;
static_assert(kIq3TileCol == kTileRows * kIq3TileBlock, "tile column = 64 tile-layout blocks");
// A stream stage column in LDS: the index bytes at the column's layout, then
// for each wavefront G a private run of kIq3Own bytes (its sign bytes, its
// scale bytes, its own copy of the column's d) that only it copies and reads,
// so the stream engine's tile-layout stages need no workgroup barrier.
constexpr int kIq3Own = 512 + 64 + 128;

template <int W, int R, bool TL>
struct Iq3Cfg {
    static constexpr int kBps = W / 4;                   // super-blocks per stage
    static constexpr int kWin = 112;                     // bytes per row window
    // one super-block of a tile (tile layout: the index bytes, then the four
    // quant-chunk wavefronts' private runs)
    static constexpr int kCol = TL ? kIq3TileSigns + 4 * kIq3Own : kTileRows * kWin;
    static constexpr int kSlot = kBps * kCol;
    static constexpr int kTable = 32768;                 // at LDS address 0
    static constexpr int kGrid = kTable;                 // staged fp32 grid, 4 KB
    static constexpr int kRing = kGrid + 256 * 16;
    static constexpr int kRed = kRing + R * kSlot;       // [2][W][64] fp32 row sums
    static constexpr int kLds = kRed + 2 * W * 64 * 4;
    // copy instructions per wavefront and stage (tile layout: the indices, then
    // the private run)
    static constexpr int kCps = 2;
};

// One work item as a cursor sees it.
struct Iq3Item {
    GemvArgs a;
    const uint8_t *sb;  // the tile's first row, rounded down to 16 bytes
    uint32_t sb_off;    // that row's offset from sb (0..15)
    uint32_t lo;        // first 16-byte granule wholly inside the weights, relative to sb (>= 0)
    uint32_t hi;        // last one (capped; the tile's granules lie far below the cap)
    int tile, split, kb0, kb1, nst, row0;
    bool head;        // holds row 0's block 0 and the buffer starts off a granule
    bool tail;        // holds the last row's last block and the buffer ends off a granule
};

template <int BPS, bool TL>
__device__ __forceinline__ void iq3_load_item(Iq3Item &it, int k, const GroupArgs &g,
                                              const GemvArgs &single) {
    int local;
    if (g.problems == nullptr) {
        it.a = single;
        local = k;
    } else {
        load_args(it.a, (cargs_p)g.problems + ((cu32_p)g.map)[k]);
        local = g.tile != nullptr ? (int)((cu32_p)g.tile)[k] : k - it.a.wg_begin;
    }
    const int splits = it.a.splits;
    if (splits == 1) {
        it.tile = local;
        it.split = 0;
        it.kb0 = 0;
        it.kb1 = it.a.nb;
    } else {
        it.tile = local / splits;
        it.split = local - it.tile * splits;
        it.kb0 = it.split * it.a.nb / splits;
        it.kb1 = (it.split + 1) * it.a.nb / splits;
    }
    it.nst = (it.kb1 - it.kb0 + BPS - 1) / BPS;
    it.row0 = it.tile * kTileRows;
    if constexpr (TL) {
        // column 0 of the tile; no partial granules anywhere in this layout
        it.sb = it.a.w + (int64_t)it.tile * it.a.nb * kIq3TileCol;
        it.sb_off = 0;
        it.lo = 0;
        it.hi = 0;
        it.head = false;
        it.tail = false;
        return;
    }
    const uintptr_t wb = (uintptr_t)it.a.w;
    const uintptr_t we = wb + (uintptr_t)it.a.n_out * (uintptr_t)it.a.row_bytes;
    const uintptr_t base0 = wb + (uintptr_t)it.row0 * (uintptr_t)it.a.row_bytes;
    const uintptr_t sb = base0 & ~(uintptr_t)15;
    it.sb = (const uint8_t *)sb;
    it.sb_off = (uint32_t)(base0 & 15);
    // The buffer holds >= 98 bytes, so wb <= lo16 < hi16 and hi16 + 16 <= we; the
    // tile's granules start at sb (>= lo16 - 16) and end below hi16 + 98 + 16.
    const uintptr_t lo16 = (wb + 15) & ~(uintptr_t)15;
    const uintptr_t hi16 = (we & ~(uintptr_t)15) - 16;
    it.lo = lo16 > sb ? (uint32_t)(lo16 - sb) : 0u;
    it.hi = hi16 - sb < 0x40000000u ? (uint32_t)(hi16 - sb) : 0x40000000u;
    it.head = (wb & 15) != 0 && it.row0 == 0 && it.kb0 == 0;
    it.tail = (we & 15) != 0 && it.row0 + kTileRows >= it.a.n_out && it.kb1 == it.a.nb;
}

// The bytes of one block that wavefront G uses, 32-bit aligned to the block:
// index bytes 16G..16G+15, sign/scale words 2G and 2G+1, and d (low 16 bits).
// From the tile layout, words[] holds the sign bytes of sub-blocks 2G and 2G+1
// (eight signs per byte) and sc their scales (low nibble 2G, high 2G+1).
struct Iq3Raw {
    uint32_t idx[4];
    uint32_t words[2];
    uint32_t d16;
    uint32_t sc;
};

// From a row window in LDS: `win` = window + (sh & 12), sh = block offset in it
// (even). Container order: the fields start at block bytes 0, 64 and 96.
template <int G>
__device__ __forceinline__ void iq3_fetch(const uint8_t *win, uint32_t sh, Iq3Raw &r) {
    const uint32_t *p = (const uint32_t *)win;
    uint32_t a[5], v[3];
#pragma unroll
    for (int i = 0; i < 5; ++i) a[i] = p[4 * G + i];
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = p[16 + 2 * G + i];
    const uint32_t dw = p[24];
#pragma unroll
    for (int i = 0; i < 4; ++i) r.idx[i] = __builtin_amdgcn_alignbyte(a[i + 1], a[i], sh);
#pragma unroll
    for (int i = 0; i < 2; ++i) r.words[i] = __builtin_amdgcn_alignbyte(v[i + 1], v[i], sh);
    r.d16 = dw >> ((sh & 2u) << 3);
}

// The same for llama.cpp's order (d at 0, indices at 2, words at 66). The index
// and word fields start (sh & 3) + 2 bytes into their dword runs: one dword on
// and aligned when sh & 2 (shift 0), else 2 bytes in (shift 2). The dword
// after each field is only needed with shift 2; the one read in its place
// with shift 0 is never used. Every read lies inside the 112-byte window: the
// last starts at window byte (sh & 12) + 96 <= 108.
template <int G>
__device__ __forceinline__ void iq3_fetch_xxs(const uint8_t *win, uint32_t sh, Iq3Raw &r) {
    const uint32_t *p = (const uint32_t *)win;
    const uint32_t up = (sh >> 1) & 1u;
    const uint32_t shift = (sh + 2u) & 3u;
    uint32_t a[5], v[3];
#pragma unroll
    for (int i = 0; i < 5; ++i) a[i] = p[4 * G + up + i];
    v[0] = p[16 + 2 * G + up];
    v[1] = p[17 + 2 * G + up];
    v[2] = p[18 + 2 * G];
#pragma unroll
    for (int i = 0; i < 4; ++i) r.idx[i] = __builtin_amdgcn_alignbyte(a[i + 1], a[i], shift);
#pragma unroll
    for (int i = 0; i < 2; ++i) r.words[i] = __builtin_amdgcn_alignbyte(v[i + 1], v[i], shift);
    r.d16 = p[0] >> ((sh & 2u) << 3);
}

// From a tile-layout column copied whole (this lane's row).
template <int G>
__device__ __forceinline__ void iq3_fetch_tiled(const uint8_t *col, int lane, Iq3Raw &r) {
    const uint4 q = *(const uint4 *)(col + G * 1024 + 16 * lane);
    const uint2 w = *(const uint2 *)(col + kIq3TileSigns + G * 512 + 8 * lane);
    r.idx[0] = q.x;
    r.idx[1] = q.y;
    r.idx[2] = q.z;
    r.idx[3] = q.w;
    r.words[0] = w.x;
    r.words[1] = w.y;
    r.sc = col[kIq3TileScales + G * 64 + lane];
    r.d16 = *(const uint16_t *)(col + kIq3TileD + 2 * lane);
}

// From a stream stage column (this lane's row; wavefront G's private run).
template <int G>
__device__ __forceinline__ void iq3_fetch_tiled_own(const uint8_t *col, int lane, Iq3Raw &r) {
    const uint4 q = *(const uint4 *)(col + G * 1024 + 16 * lane);
    const uint8_t *own = col + kIq3TileSigns + G * kIq3Own;
    const uint2 w = *(const uint2 *)(own + 8 * lane);
    r.idx[0] = q.x;
    r.idx[1] = q.y;
    r.idx[2] = q.z;
    r.idx[3] = q.w;
    r.words[0] = w.x;
    r.words[1] = w.y;
    r.sc = own[512 + lane];
    r.d16 = *(const uint16_t *)(own + 576 + 2 * lane);
}

// From global memory, 2 bytes at a time (the block is 2-byte aligned), in
// either byte order.
template <int G>
__device__ __forceinline__ void iq3_fetch_direct(const uint8_t *blk, bool xxs, Iq3Raw &r) {
    const uint16_t *h = (const uint16_t *)blk;
    const int hi = xxs ? 1 : 0, hw = xxs ? 33 : 32, hd = xxs ? 0 : 48;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.idx[i] = (uint32_t)h[hi + 8 * G + 2 * i] | ((uint32_t)h[hi + 8 * G + 2 * i + 1] << 16);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        r.words[i] = (uint32_t)h[hw + 4 * G + 2 * i] | ((uint32_t)h[hw + 4 * G + 2 * i + 1] << 16);
    r.d16 = h[hd];
}

// 8 x the low / high 16 bits of v (one v_mad_u32_u16 each).
__device__ __forceinline__ uint32_t lo16_x8(uint32_t v) {
    uint32_t r;
    asm("v_mad_u32_u16 %0, %1, 8, 0" : "=v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ uint32_t hi16_x8(uint32_t v) {
    uint32_t r;
    asm("v_mad_u32_u16 %0, %1, 8, 0 op_sel:[1,0,0,0]" : "=v"(r) : "v"(v));
    return r;
}

// The sign-folded table entries of the eight 4-weight groups of sub-block
// half of the chunk: group k's entry (nibble*256 + index byte) * 8, its index
// byte k & 3 of word idx[2 half + k / 4], its sign nibble byte k / 2 of ne
// (k even) or no (k odd). One v_perm forms the entry numbers of groups k and
// k + 2 in the two 16-bit halves (same index word, same nibble word), and one
// multiply-add per half scales each to a byte address: three VALU ops per two
// groups instead of a perm and a shift per group.
__device__ __forceinline__ void iq3_table_reads(const Iq3Raw &r, int half, uint32_t ne,
                                                uint32_t no, u32x2 (&v)[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int k = (p & 1) | ((p & 2) << 1);   // 0, 1, 4, 5
        const uint32_t sel = (uint32_t)(k & 3) | ((uint32_t)(4 + (k >> 1)) << 8) |
                             ((uint32_t)((k + 2) & 3) << 16) | ((uint32_t)(4 + ((k + 2) >> 1)) << 24);
        const uint32_t pr = __builtin_amdgcn_perm((k & 1) ? no : ne, r.idx[2 * half + (k >> 2)], sel);
        v[k] = lds_load<u32x2>(lo16_x8(pr));
        v[k + 2] = lds_load<u32x2>(hi16_x8(pr));
    }
}

// acc + sum over wavefront G's 64 weights of this lane's row of w*x.
// xg: x[256*b + 64*G] (wave-uniform). The sign-folded grid table sits at LDS
// address 0. Two interleaved partial sums per sub-block keep consecutive FMAs
// independent. SX: the raw block comes from the tile layout (signs written
// out, scales apart).
template <int G, bool SX>
__device__ __forceinline__ float iq3_dot(const Iq3Raw &r, cfloat_p xg, float acc) {
    const float dq = h2f_lo(r.d16) * 0.25f;   // d*(0.5+code)*0.5 == (d/4)*(2*code+1), exact
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t word = r.words[half];
        const uint32_t s8 = SX ? word : iq3_signs(word);
        const uint32_t code = SX ? (r.sc >> (4 * half)) & 15u : word >> 28;
        // sign nibble of 4-weight group k: low nibble of byte k/2 of ne (k even) or no (k odd)
        const uint32_t ne = s8 & 0x0F0F0F0Fu;
        const uint32_t no = (s8 >> 4) & 0x0F0F0F0Fu;
        const float db = dq * (float)(2u * code + 1u);
        const cfloat_p xs = xg + 32 * half;
        // All eight table reads and the 32 activations (scalar loads) are issued
        // before the first FMA: LDS and scalar loads share one wait counter, and
        // interleaved (as the compiler schedules them otherwise) every pair of
        // reads waited out a full round trip (measured: tile-layout stream
        // 95 -> 93 us, row-major 138 -> 132 us).
        u32x2 v[8];
        iq3_table_reads(r, half, ne, no, v);
        float xv[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) xv[i] = xs[i];
        __builtin_amdgcn_sched_barrier(0);
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s0 = __builtin_fmaf(h2f_lo(v[k].x), xv[4 * k + 0], s0);
            s1 = __builtin_fmaf(h2f_hi(v[k].x), xv[4 * k + 1], s1);
            s0 = __builtin_fmaf(h2f_lo(v[k].y), xv[4 * k + 2], s0);
            s1 = __builtin_fmaf(h2f_hi(v[k].y), xv[4 * k + 3], s1);
        }
        acc = __builtin_fmaf(db, s0 + s1, acc);
    }
    return acc;
}

template <typename T>
__device__ __forceinline__ void lds_store(uint32_t addr, T v) {
    *(__attribute__((address_space(3))) T *)(size_t)addr = v;
}

// Entries (s, i), s = s0, s0 + ds, ... < 16, of the sign-folded table from
// grid row g: the four fp16 magnitudes converted once, each sign pattern made
// by flipping their sign bits (conversion to fp16 rounds symmetrically, so
// this is the fp16 of each signed value). Measured against converting every
// entry: IQ3 5632 x 2048 on row groups (16 entries per thread) 6.12 -> 5.96 us.
__device__ __forceinline__ void iq3_table_row(int i, float4 g, int s0, int ds) {
    const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)g.x);
    const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)g.y);
    const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)g.z);
    const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)g.w);
    const uint32_t lo = h0 | (h1 << 16), hi = h2 | (h3 << 16);
    for (int s = s0; s < 16; s += ds) {
        const uint32_t mlo = ((uint32_t)(s & 1) << 15) | ((uint32_t)(s & 2) << 30);
        const uint32_t mhi = ((uint32_t)(s & 4) << 13) | ((uint32_t)(s & 8) << 28);
        const u32x2 e = {lo ^ mlo, hi ^ mhi};
        lds_store<u32x2>(s * 2048 + i * 8, e);
    }
}

template <int G, int W, int R, bool TL>
__device__ __forceinline__ void iq3_stream(const GroupArgs &g, const GemvArgs &single,
                                           const float *grid, int nitems, uint8_t *smem) {
    static_assert(R >= 2 && R <= 4, "ring of two to four stages");
    using C = Iq3Cfg<W, R, TL>;
    constexpr int BPS = C::kBps;
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const int wave = 4 * j + G;
    const int stride = gridDim.x;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    int kc = skip_holes(blockIdx.x, stride, nitems, g);  // item being computed
    if (kc >= nitems) return;

    // Wavefronts 0..3 stage the grid's 4 KB (lane l of wavefront w: bytes
    // 16*(64w + l)) ahead of any stage copy, so waiting for it leaves those in flight.
    if (wave < 4)
        dma16((const uint8_t *)grid + 16 * (64 * wave + lane), lds0 + C::kGrid + 1024 * wave);

    // This wavefront's copy lanes: granule k = 64i + lane (k < 112) of its 16
    // rows, i.e. granule k%7 of the window of row 16G + k/7, which lands at
    // LDS byte 16k of the wavefront's quarter of the block column.
    int crow[2];
    uint32_t cgran[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int k = min(64 * i + lane, 111);
        crow[i] = 16 * G + k / 7;
        cgran[i] = 16u * (uint32_t)(k % 7);
    }

    Iq3Item c;
    iq3_load_item<BPS, TL>(c, kc, g, single);

    // copy cursor: next stage sd of item kd goes to ring slot slot_d
    int kd = kc, sd = 0, slot_d = 0, pending = 0;
    Iq3Item d = c;
    uint32_t doff[2];  // this lane's granule of block 0 of its row, relative to d.sb (< 2 MB)
    auto prep_copy = [&]() {
        if constexpr (TL) return;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            doff[i] = d.sb_off +
                      (uint32_t)(min(d.row0 + crow[i], d.a.n_out - 1) - d.row0) *
                          (uint32_t)d.a.row_bytes +
                      cgran[i];
    };
    // Tile layout: wavefront G copies its index bytes (1 KB, every lane) and
    // its private run (lanes 0..31 its sign bytes, 32..35 its scale bytes,
    // 36..43 the column's d): every byte a wavefront reads in a stage is one it
    // copied, so stages need no workgroup barrier, only the wavefront's own
    // wait for its copies.
    const uint32_t t_off0 = (uint32_t)(G * 1024 + 16 * lane);
    const uint32_t t_off1 =
        lane < 32 ? (uint32_t)(kIq3TileSigns + G * 512 + 16 * lane)
                  : lane < 36 ? (uint32_t)(kIq3TileScales + G * 64 + 16 * (lane - 32))
                              : (uint32_t)(kIq3TileD + 16 * (lane - 36));
    prep_copy();
    uint32_t flags = 0;  // bit k: this wavefront's copies are in ring slot k
    auto issue_next = [&]() {
        if (kd >= nitems) return;
        const int b = d.kb0 + sd * BPS + j;
        if (b < d.kb1) {
            if constexpr (TL) {
                const uint32_t colb = lds0 + C::kRing + slot_d * C::kSlot + j * C::kCol;
                const uint8_t *src = d.sb + (int64_t)b * kIq3TileCol;
                dma16_stream(src + t_off0, colb + G * 1024);
                if (lane < kIq3Own / 16) dma16_stream(src + t_off1, colb + kIq3TileSigns + G * kIq3Own);
            } else {
                const uint32_t base =
                    lds0 + C::kRing + slot_d * C::kSlot + j * C::kCol + G * (16 * C::kWin);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (i == 0 || lane < 48) {
                        // (offset + a multiple of 16) & ~15 keeps the granule index
                        const uint32_t off = min(max((doff[i] + (uint32_t)(kIq3Bytes * b)) & ~15u, d.lo), d.hi);
                        dma16(d.sb, off, base + 1024 * i);
                    }
                }
            }
            flags |= 1u << slot_d;
        } else {
            flags &= ~(1u << slot_d);
        }
        ++pending;
        slot_d = slot_d + 1 == R ? 0 : slot_d + 1;
        if (++sd == d.nst) {
            sd = 0;
            kd = skip_holes(kd + stride, stride, nitems, g);
            if (kd < nitems) {
                iq3_load_item<BPS, TL>(d, kd, g, single);
                prep_copy();
            }
        }
    };
#pragma unroll
    for (int i = 0; i < R - 1; ++i) issue_next();

    // Grid staged (this wavefront's part: its stage copies, two per stage, may
    // stay in flight), then the sign-folded table from it. A grid value that
    // fp16 cannot hold would be rounded in the table: the workgroup then
    // stores NaN in every row instead (host code that creates a group rejects
    // such a grid up front). The vote goes through a word of the row-sum
    // buffer, idle until the first item ends.
    volatile uint32_t *vote = (volatile uint32_t *)(smem + C::kRed);
    if (threadIdx.x == 0) *vote = 0u;
    if (wave < 4) wait_vmcnt_upto(C::kCps * __builtin_popcount(flags));
    lds_barrier();
    {
        const int t = threadIdx.x;
        const int i = t & 255;
        const float4 gv = *(const float4 *)(smem + C::kGrid + 16 * i);
        iq3_table_row(i, gv, t >> 8, W / 4);
        const bool exact =
            fp16_exact(gv.x) && fp16_exact(gv.y) && fp16_exact(gv.z) && fp16_exact(gv.w);
        if (__builtin_amdgcn_ballot_w64(!exact) != 0 && lane == 0) *vote = 1u;
    }
    lds_barrier();
    const bool grid_bad = __builtin_amdgcn_readfirstlane(*vote) != 0u;

    float *red = (float *)(smem + C::kRed);
    int slot_c = 0;
    int parity = 0;   // row-sum buffer of this item (two, alternating)
    for (;;) {
        const int row = c.row0 + lane;
        // low bits of this lane's row address (block offsets within granules)
        const uint32_t rlo = (uint32_t)(uintptr_t)c.a.w +
                             (uint32_t)min(row, c.a.n_out - 1) * (uint32_t)c.a.row_bytes;
        float acc = 0.0f;
        for (int s = 0; s < c.nst; ++s) {
            // Copies of the stages after this one may stay in flight.
            const int nxt = slot_c + 1 == R ? 0 : slot_c + 1;
            int younger = 0;
            if (R >= 3 && pending > 1) younger += C::kCps * (int)((flags >> nxt) & 1u);
            if (R >= 4 && pending > 2) younger += C::kCps * (int)((flags >> (nxt + 1 == R ? 0 : nxt + 1)) & 1u);
            wait_vmcnt_upto(younger);
            if constexpr (TL) {
                // this wavefront's own copies of the stage are in; its reads of
                // the slot refilled below (the previous step's) are complete
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            } else {
                lds_barrier();   // stage in slot_c complete for every wavefront (and the table)
            }
            issue_next();    // refill the slot computed in the previous step
            const int b = c.kb0 + s * BPS + j;
            if (TL && b < c.kb1) {
                Iq3Raw raw;
                iq3_fetch_tiled_own<G>(smem + C::kRing + slot_c * C::kSlot + j * C::kCol, lane, raw);
                acc = iq3_dot<G, true>(raw, as_scalar(c.a.x) + (int64_t)kQK * b + 64 * G, acc);
            } else if (b < c.kb1) {
                const uint32_t sh = (rlo + (uint32_t)(kIq3Bytes * b)) & 15u;
                const uint8_t *win = smem + C::kRing + slot_c * C::kSlot + j * C::kCol +
                                     lane * C::kWin + (sh & 12u);
                const bool xxs = c.a.layout == kLayoutRowsXxs;
                Iq3Raw raw;
                if (xxs)
                    iq3_fetch_xxs<G>(win, sh, raw);
                else
                    iq3_fetch<G>(win, sh, raw);
                const bool head = c.head && b == 0;
                const bool tail = c.tail && b == c.a.nb - 1;
                if (head || tail) {   // wave-uniform, at most twice per matrix
                    if ((head && row == 0) || (tail && row == c.a.n_out - 1))
                        iq3_fetch_direct<G>(c.a.w + (int64_t)row * c.a.row_bytes + kIq3Bytes * b,
                                            xxs, raw);
                }
                acc = iq3_dot<G, false>(raw, as_scalar(c.a.x) + (int64_t)kQK * b + 64 * G, acc);
            }
            --pending;
            slot_c = nxt;
        }
        // row sums of the W wavefronts, in wavefront order (two buffers: with no
        // barrier between stages, a wavefront can reach the next item's end
        // while wavefront 0 still reads this one's)
        float *rb = red + parity * W * 64;
        parity ^= 1;
        rb[wave * 64 + lane] = acc;
        lds_barrier();
        if (wave == 0) {
            float tsum = rb[lane];
            for (int w = 1; w < W; ++w) tsum += rb[w * 64 + lane];
            if (grid_bad) tsum = __builtin_nanf("");
            const float total[1] = {tsum};
            tile_epilogue<1>(c.a, c.tile, c.split, total);
        }
        kc = skip_holes(kc + stride, stride, nitems, g);
        if (kc >= nitems) break;
        iq3_load_item<BPS, TL>(c, kc, g, single);
    }
}

template <int W, int R, bool TL>
__global__ __launch_bounds__(W * 64) void iq3_stream_kernel(GroupArgs g, GemvArgs single,
                                                            const float *grid, int nitems) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    switch (__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3)) {
        case 0: iq3_stream<0, W, R, TL>(g, single, grid, nitems, smem); break;
        case 1: iq3_stream<1, W, R, TL>(g, single, grid, nitems, smem); break;
        case 2: iq3_stream<2, W, R, TL>(g, single, grid, nitems, smem); break;
        default: iq3_stream<3, W, R, TL>(g, single, grid, nitems, smem); break;
    }
}

// Resident workgroups of one kernel variant on the current device (cached).
template <int W, int R, bool TL>
int iq3_slots() {
    // a function-local static: initialised once even under concurrent first calls
    static const int slots = [] {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        constexpr size_t lds = Iq3Cfg<W, R, TL>::kLds;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, iq3_stream_kernel<W, R, TL>,
                                                         W * 64, lds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        return per_cu * cus;
    }();
    return slots;
}

template <int W, int R>
hipError_t iq3_launch(const GroupArgs &g, const GemvArgs &single, const float *grid, int nitems,
                      bool tiled, hipStream_t s) {
    int n = tiled ? iq3_slots<W, R, true>() : iq3_slots<W, R, false>();
    if (n > nitems) n = nitems;
    if (tiled) {
        constexpr size_t lds = Iq3Cfg<W, R, true>::kLds;
        hipLaunchKernelGGL((iq3_stream_kernel<W, R, true>), dim3((unsigned)n), dim3(W * 64), lds, s,
                           g, single, grid, nitems);
    } else {
        constexpr size_t lds = Iq3Cfg<W, R, false>::kLds;
        hipLaunchKernelGGL((iq3_stream_kernel<W, R, false>), dim3((unsigned)n), dim3(W * 64), lds,
                           s, g, single, grid, nitems);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ short calls
//
// A single IQ3 GEMV of a few MB (the short-call scheme of short.hip): each
// 64-row tile's super-blocks are split over S workgroups (tiles x S <= compute
// units), a workgroup holds C <= kShortMaxBlocks columns with four wavefronts
// per column (wavefront 4j + G: quant chunk G of column j), and every byte a
// workgroup needs is requested at its start: the fp32 grid (4 KB, first), each
// column (row-major: the seven 16-byte granules of each row's block window,
// clamped into the buffer as in the stream engine; tile layout: the 6272-byte
// column), the activations as scalar loads. The sign-folded table of the
// stream engine is built while the columns are in flight: the grid arrives
// from L2 well before them, so waiting for it leaves the columns' copies
// outstanding (per-wavefront memory counters complete in order). A version
// that read the fp32 grid rows and flipped the signs per weight instead of the
// table (no build, 16-byte LDS reads, three more VALU ops per weight) took
// 7.8 / 7.1 us for the two 4.4 MB shapes of the IQ3 configuration.
constexpr int kIq3ShortGrid = 32768;   // staged fp32 grid [256][4], after the table
constexpr int kIq3ShortVote = kIq3ShortGrid + 4096;    // grid-exactness vote
constexpr int kIq3ShortCols = kIq3ShortVote + 16;      // columns (16-byte aligned)
constexpr int iq3_short_col(bool tl) { return tl ? kIq3TileCol : kTileRows * 112; }
constexpr int iq3_short_lds(int c, bool tl) {
    return kIq3ShortCols + c * iq3_short_col(tl) + 4 * c * kTileRows * 4;
}

// iq3_dot with the chunk's 64 activations already in registers.
template <int G, bool SX, typename XAt>
__device__ __forceinline__ float iq3_dot_regs(const Iq3Raw &r, XAt xat, float acc) {
    const float dq = h2f_lo(r.d16) * 0.25f;   // d*(0.5+code)*0.5 == (d/4)*(2*code+1), exact
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t word = r.words[half];
        const uint32_t s8 = SX ? word : iq3_signs(word);
        const uint32_t ne = s8 & 0x0F0F0F0Fu;
        const uint32_t no = (s8 >> 4) & 0x0F0F0F0Fu;
        const uint32_t code = SX ? (r.sc >> (4 * half)) & 15u : word >> 28;
        const float db = dq * (float)(2u * code + 1u);
        u32x2 v[8];
        iq3_table_reads(r, half, ne, no, v);
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s0 = __builtin_fmaf(h2f_lo(v[k].x), xat(32 * half + 4 * k + 0), s0);
            s1 = __builtin_fmaf(h2f_hi(v[k].x), xat(32 * half + 4 * k + 1), s1);
            s0 = __builtin_fmaf(h2f_lo(v[k].y), xat(32 * half + 4 * k + 2), s0);
            s1 = __builtin_fmaf(h2f_hi(v[k].y), xat(32 * half + 4 * k + 3), s1);
        }
        acc = __builtin_fmaf(db, s0 + s1, acc);
    }
    return acc;
}

template <int G>
__device__ __forceinline__ void iq3_short_fetch(const uint8_t *col, int layout, uint32_t sh,
                                                int lane, Iq3Raw &r) {
    if (layout == kLayoutTiles)
        iq3_fetch_tiled<G>(col, lane, r);
    else if (layout == kLayoutRowsXxs)
        iq3_fetch_xxs<G>(col + 112 * lane + (sh & 12u), sh, r);
    else
        iq3_fetch<G>(col + 112 * lane + (sh & 12u), sh, r);
}

template <int G>
__device__ __forceinline__ float iq3_short_column(const GemvArgs &a, const uint8_t *col, int row,
                                                  int b, int lane, const float (&xs)[64]) {
    const bool tl = a.layout == kLayoutTiles;
    const uintptr_t wb = (uintptr_t)a.w;
    const uintptr_t we = wb + (uintptr_t)a.n_out * (uintptr_t)a.row_bytes;
    const uintptr_t start = wb + (uintptr_t)min(row, a.n_out - 1) * (uintptr_t)a.row_bytes +
                            (uintptr_t)kIq3Bytes * b;
    Iq3Raw raw;
    iq3_short_fetch<G>(col, a.layout, (uint32_t)start & 15u, lane, raw);
    if (tl) return iq3_dot_regs<G, true>(raw, [&](int i) { return xs[i]; }, 0.0f);
    // a window granule that lies partly outside the buffer was clamped: that
    // row's block comes from 2-byte loads instead (at most twice per matrix)
    const bool head = (wb & 15) != 0 && row == 0 && b == 0;
    const bool tail = (we & 15) != 0 && row == a.n_out - 1 && b == a.nb - 1;
    if (head || tail)
        iq3_fetch_direct<G>(a.w + (int64_t)row * a.row_bytes + kIq3Bytes * b,
                            a.layout == kLayoutRowsXxs, raw);
    return iq3_dot_regs<G, false>(raw, [&](int i) { return xs[i]; }, 0.0f);
}

template <int C>
__global__ __launch_bounds__(256 * C) void iq3_short_kernel(GemvArgs a, ShortState st,
                                                            const float *grid) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int W = 4 * C;
    const bool tl = a.layout == kLayoutTiles;
    const int colsz = tl ? kIq3TileCol : kTileRows * 112;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = wave >> 2;
    const int G = wave & 3;
    int tile, split;
    if (!short_item(a, tile, split)) return;
    const int kb0 = split * a.nb / a.splits;
    const int kb1 = (split + 1) * a.nb / a.splits;
    const bool live = kb0 + j < kb1;
    const int b = kb0 + j;
    const int row = tile * kTileRows + lane;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t colb = lds0 + kIq3ShortCols + j * colsz;

    // The tile's epoch (split launches; used at the end), the grid (wavefronts
    // 0..3, 1 KB each), then the columns: copies G and G + 4 of each column's
    // seven 1 KB pieces (the last one 384 bytes on the tile layout).
    uint32_t epoch = 0;
    if (a.splits > 1 && wave == 0)
        epoch = __hip_atomic_load(&st.epochs[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave < 4) dma16((const uint8_t *)grid + 16 * (64 * wave + lane), lds0 + kIq3ShortGrid + 1024 * wave);
    int ncopy = 0;
    if (live) {
        const uintptr_t wb = (uintptr_t)a.w;
        const uintptr_t we = wb + (uintptr_t)a.n_out * (uintptr_t)a.row_bytes;
        const uintptr_t lo16 = (wb + 15) & ~(uintptr_t)15;    // first whole granule
        const uintptr_t hi16 = (we & ~(uintptr_t)15) - 16;    // last whole granule
        for (int q = G; q < 7; q += 4) {
            const uint32_t dst = colb + 1024 * q;
            if (tl) {
                if (q < 6 || lane < (kIq3TileCol - 6144) / 16)
                    dma16(a.w + ((int64_t)tile * a.nb + b) * kIq3TileCol + 1024 * q + 16 * lane, dst);
            } else {
                const int k = 64 * q + lane;          // granule k % 7 of row k / 7's window
                const int r = tile * kTileRows + k / 7;
                const uintptr_t start = wb + (uintptr_t)min(r, a.n_out - 1) * (uintptr_t)a.row_bytes +
                                        (uintptr_t)kIq3Bytes * b;
                uintptr_t gaddr = (start & ~(uintptr_t)15) + 16 * (uintptr_t)(k % 7);
                gaddr = gaddr < lo16 ? lo16 : (gaddr > hi16 ? hi16 : gaddr);
                dma16((const void *)gaddr, dst);
            }
            ++ncopy;
        }
    }
    const int xb = live ? b : kb0;
    const cfloat_p xg = as_scalar(a.x) + (int64_t)kQK * xb + 64 * G;
    float xs[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) xs[i] = xg[i];
    volatile __attribute__((address_space(3))) uint32_t *vote =
        (volatile __attribute__((address_space(3))) uint32_t *)(size_t)(lds0 + kIq3ShortVote);
    if (threadIdx.x == 0) *vote = 0u;

    // The grid is in LDS once this wavefront's column copies (issued after it)
    // are the only ones outstanding.
    if (wave < 4) wait_vmcnt_upto(ncopy);
    lds_barrier();
    {
        const int t = threadIdx.x;
        const int i = t & 255;
        const f32x4 gv = lds_load<f32x4>(kIq3ShortGrid + 16 * i);
        const float4 g4 = {gv[0], gv[1], gv[2], gv[3]};
        iq3_table_row(i, g4, t >> 8, W / 4);
        const bool exact = fp16_exact(gv[0]) && fp16_exact(gv[1]) && fp16_exact(gv[2]) && fp16_exact(gv[3]);
        if (__builtin_amdgcn_ballot_w64(!exact) != 0 && lane == 0) *vote = 1u;
    }
    wait_vmcnt<0>();
    lds_barrier();   // the columns and the table

    float acc = 0.0f;
    if (live) {
        const uint8_t *col = smem + (colb - lds0);
        switch (G) {
            case 0: acc = iq3_short_column<0>(a, col, row, b, lane, xs); break;
            case 1: acc = iq3_short_column<1>(a, col, row, b, lane, xs); break;
            case 2: acc = iq3_short_column<2>(a, col, row, b, lane, xs); break;
            default: acc = iq3_short_column<3>(a, col, row, b, lane, xs); break;
        }
    }
    float *red = (float *)(smem + kIq3ShortCols + C * colsz);
    red[wave * 64 + lane] = acc;
    lds_barrier();
    if (wave != 0) return;
    float total = red[lane];
    for (int w = 1; w < W; ++w) total += red[w * 64 + lane];
    if (*vote != 0u) total = __builtin_nanf("");
    // (the epoch's first use: the compiler's wait for its load goes here, not
    // ahead of the table build)
    asm volatile("" : "+v"(epoch));
    short_epilogue(a, st, tile, split, epoch, total);
}

// ------------------------------------------------------------------ row groups
//
// Rows of at most 24 blocks (n_in <= 6144) on the short-call matrices: a
// workgroup of 4 NS wavefronts takes eight whole rows, so no split sums meet
// through memory (the Q4_K row-group kernel's scheme). Wavefront w takes
// quant chunk w % 4 of the blocks of set w / 4, lane r + 8s row r's block
// s + 8 (w / 4), with its 64 activations in registers (sixteen 16-byte loads).
// Each thread loads one grid row into registers and builds its table entries
// from it as soon as it arrives. Measured (kernel trace, cold weights) against
// the split kernel: 5632 x 2048 (NS = 1) 7.20 -> 5.92 us, 2048 x 5632 (NS = 3)
// 6.60 -> 6.36 us.
// The rows arrive as one contiguous run of 16-byte granules (row-major, either
// byte order: 8 x nb x 98 bytes from the group's first block, granules that
// reach outside the buffer clamped and the two blocks they hold read directly
// as in the stream engine) or as the eight rows' slices of each tile-layout
// column (848 bytes: index, sign, scale and d runs; the scale runs are the
// 16-byte granules that hold the rows' 8 bytes). The sign-folded table and the
// exactness vote are the short-call kernel's.
constexpr int kIq3RgRows = 8;
constexpr int kIq3RgMaxBlocks = 24;
constexpr int kIq3RgGran = 53;                          // granules of one slice
constexpr int kIq3RgSlice = 16 * kIq3RgGran;            // 8 rows of a tile-layout column
// The rows' granules (row-major run with its head and one over-read granule,
// or the tile slices), in whole 64-granule copy instructions; then the
// reduction [wavefronts][8 rows] fp32.
__host__ __device__ constexpr int iq3_rg_region(int nb) {
    const int run = (15 + kIq3RgRows * nb * kIq3Bytes + 15) / 16 + 1;
    const int gr = run > kIq3RgGran * nb ? run : kIq3RgGran * nb;
    return (gr + 63) / 64 * 64 * 16;
}
__host__ __device__ constexpr int iq3_rg_lds(int nb, int waves) {
    return kIq3ShortCols + iq3_rg_region(nb) + waves * kIq3RgRows * 4;
}
static_assert(iq3_rg_lds(kIq3RgMaxBlocks, 12) <= 65536, "LDS of one workgroup");

// Byte offset in a tile-layout column of granule g (0..52) of the eight-row
// slice starting at row rit (a multiple of 8): index runs, sign runs, the
// granule of each scale run that holds the rows' bytes (at byte rit & 8), d.
__device__ __forceinline__ int iq3_rg_tile_off(int g, int rit) {
    if (g < 32) return (g >> 3) * 1024 + 16 * rit + 16 * (g & 7);
    if (g < 48) return kIq3TileSigns + ((g - 32) >> 2) * 512 + 8 * rit + 16 * ((g - 32) & 3);
    if (g < 52) return kIq3TileScales + (g - 48) * 64 + (rit & ~15);
    return kIq3TileD + 2 * rit;
}

template <int G>
__device__ __forceinline__ float iq3_rows_dot(const GemvArgs &a, const uint8_t *rg, uint32_t o,
                                              int row, int b, int r, const f32x4 (&xv)[16]) {
    Iq3Raw raw;
    if (a.layout == kLayoutTiles) {
        const uint8_t *sl = rg + b * kIq3RgSlice;
        const uint4 q = *(const uint4 *)(sl + G * 128 + 16 * r);
        const uint2 w = *(const uint2 *)(sl + 512 + G * 64 + 8 * r);
        raw.idx[0] = q.x;
        raw.idx[1] = q.y;
        raw.idx[2] = q.z;
        raw.idx[3] = q.w;
        raw.words[0] = w.x;
        raw.words[1] = w.y;
        raw.sc = sl[768 + G * 16 + (row & 8) + r];
        raw.d16 = *(const uint16_t *)(sl + 832 + 2 * r);
        return iq3_dot_regs<G, true>(raw, [&](int i) { return xv[i >> 2][i & 3]; }, 0.0f);
    } else {
        const bool xxs = a.layout == kLayoutRowsXxs;
        const uint8_t *win = rg + (o & ~3u);
        if (xxs)
            iq3_fetch_xxs<G>(win, o, raw);
        else
            iq3_fetch<G>(win, o, raw);
        const uintptr_t wb = (uintptr_t)a.w;
        const uintptr_t we = wb + (uintptr_t)a.n_out * (uintptr_t)a.row_bytes;
        const bool head = (wb & 15) != 0 && row == 0 && b == 0;
        const bool tail = (we & 15) != 0 && row == a.n_out - 1 && b == a.nb - 1;
        if (head || tail) iq3_fetch_direct<G>(a.w + (int64_t)row * a.row_bytes + kIq3Bytes * b, xxs, raw);
    }
    return iq3_dot_regs<G, false>(raw, [&](int i) { return xv[i >> 2][i & 3]; }, 0.0f);
}

template <int NS>
__global__ __launch_bounds__(256 * NS) void iq3_rows_kernel(GemvArgs a, const float *grid) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int R = kIq3RgRows;
    constexpr int W = 4 * NS;          // block set wave / 4, chunk wave % 4
    const bool tl = a.layout == kLayoutTiles;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = wave & 3;
    const int nb = a.nb;
    const int row0 = blockIdx.x * R;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t rgb = lds0 + kIq3ShortCols;
    const int r = lane & (R - 1);
    const int b = (lane >> 3) + 8 * (wave >> 2);

    // This thread's grid row (its table entries), then the activations, then
    // the rows' copies: the table is built as soon as the grid row is in, with
    // no barrier before it.
    const f32x4 gv = *(const f32x4 *)(grid + 4 * (threadIdx.x & 255));
    __builtin_amdgcn_sched_barrier(0);   // (kept the oldest load: its wait then lets the rest fly)
    f32x4 xv[16];
    {
        const f32x4 *xp = (const f32x4 *)(a.x + (int64_t)kQK * min(b, nb - 1) + 64 * G);
#pragma unroll
        for (int q = 0; q < 16; ++q) xv[q] = xp[q];
    }
    uint32_t o0 = 0;   // the group's first block in the copied run (row-major)
    if (tl) {
        const int nk = kIq3RgGran * nb;
        const int rit = row0 & 63;
        for (int k0 = 64 * wave; k0 < nk; k0 += 64 * W) {
            const int k = min(k0 + lane, nk - 1);
            const int bb = k / kIq3RgGran;
            dma16(a.w + ((int64_t)(row0 >> 6) * nb + bb) * kIq3TileCol +
                      iq3_rg_tile_off(k - kIq3RgGran * bb, rit),
                  rgb + 16 * k0);
        }
    } else {
        const uintptr_t wb = (uintptr_t)a.w;
        const uintptr_t we = wb + (uintptr_t)a.n_out * (uintptr_t)a.row_bytes;
        const uintptr_t lo16 = (wb + 15) & ~(uintptr_t)15;   // first whole granule
        const uintptr_t hi16 = (we & ~(uintptr_t)15) - 16;   // last whole granule
        const uintptr_t start = wb + (uintptr_t)row0 * (uintptr_t)a.row_bytes;
        const uintptr_t base16 = start & ~(uintptr_t)15;
        o0 = (uint32_t)(start & 15);
        const int ngr = (int)((o0 + (uint32_t)(R * a.row_bytes) + 15) / 16) + 1;
        for (int k0 = 64 * wave; k0 < ngr; k0 += 64 * W) {
            uintptr_t g = base16 + 16 * (uintptr_t)(k0 + lane);
            g = g < lo16 ? lo16 : (g > hi16 ? hi16 : g);
            dma16((const void *)g, rgb + 16 * k0);
        }
    }
    // Sign-folded table (grid row threadIdx.x); each wavefront's exactness
    // vote in a word of its own.
    {
        const float4 g4 = {gv[0], gv[1], gv[2], gv[3]};
        iq3_table_row(threadIdx.x & 255, g4, NS == 1 ? 0 : (int)(threadIdx.x >> 8), NS);
        const bool exact = fp16_exact(gv[0]) && fp16_exact(gv[1]) && fp16_exact(gv[2]) && fp16_exact(gv[3]);
        const bool any = __builtin_amdgcn_ballot_w64(!exact) != 0;
        if (wave < 4 && lane == 0)
            *(volatile __attribute__((address_space(3))) uint32_t *)(size_t)(lds0 + kIq3ShortVote + 4 * wave) = any ? 1u : 0u;
    }
    wait_vmcnt<0>();
    lds_barrier();   // the rows and the table

    float acc = 0.0f;
    const int row = row0 + r;
    if (b < nb) {
        const uint8_t *rg = smem + kIq3ShortCols;
        const uint32_t o = o0 + (uint32_t)((r * nb + b) * kIq3Bytes);
        switch (G) {
            case 0: acc = iq3_rows_dot<0>(a, rg, o, row, b, r, xv); break;
            case 1: acc = iq3_rows_dot<1>(a, rg, o, row, b, r, xv); break;
            case 2: acc = iq3_rows_dot<2>(a, rg, o, row, b, r, xv); break;
            default: acc = iq3_rows_dot<3>(a, rg, o, row, b, r, xv); break;
        }
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    float *red = (float *)(smem + kIq3ShortCols + iq3_rg_region(nb));
    if (lane < R) red[wave * R + lane] = acc;
    lds_barrier();
    if (wave != 0 || lane >= R) return;
    float total = red[lane];
#pragma unroll
    for (int w = 1; w < W; ++w) total += red[w * R + lane];
    const volatile __attribute__((address_space(3))) uint32_t *vote =
        (const volatile __attribute__((address_space(3))) uint32_t *)(size_t)(lds0 + kIq3ShortVote);
    if ((vote[0] | vote[1] | vote[2] | vote[3]) != 0u) total = __builtin_nanf("");
    if (row0 + lane < a.n_out) a.y[row0 + lane] = total;
}

// Row-major IQ3 weights -> tile layout, one workgroup per (tile, block column),
// one 4-byte unit of the column per thread and step (the source blocks are
// only 2-byte aligned: 2-byte loads). Index bytes and d are copied; each sign
// word becomes its four sign bytes (iq3_signs) and its scale nibble moves to
// the scale run.
__device__ __forceinline__ uint32_t iq3_ld32(const uint8_t *p) {
    const uint16_t *h = (const uint16_t *)p;
    return (uint32_t)h[0] | ((uint32_t)h[1] << 16);
}

__global__ __launch_bounds__(256) void iq3_pack_tiles_kernel(const uint8_t *__restrict__ src,
                                                             uint8_t *__restrict__ dst, int nb,
                                                             int n_out, bool xxs) {
    const Iq3Order fo = iq3_order(xxs);
    const int b = blockIdx.x % nb;
    const int tile = blockIdx.x / nb;
    const int64_t row_bytes = (int64_t)nb * kIq3Bytes;
    // block b of tile row rr, or null past n_out (zero blocks)
    auto blk = [&](int rr) -> const uint8_t * {
        const int r = tile * kTileRows + rr;
        return r < n_out ? src + r * row_bytes + (int64_t)b * kIq3Bytes : nullptr;
    };
    uint32_t *out = (uint32_t *)(dst + (int64_t)blockIdx.x * kIq3TileCol);
    for (int u = threadIdx.x; u < kIq3TileCol / 4; u += blockDim.x) {
        const int o = 4 * u;
        uint32_t v = 0;
        if (o < kIq3TileSigns) {            // [G][row][16] index bytes
            const uint8_t *p = blk((o & 1023) >> 4);
            if (p) v = iq3_ld32(p + fo.idx + 16 * (o >> 10) + (o & 15));
        } else if (o < kIq3TileScales) {    // [G][row][8] sign bytes of words 2G, 2G+1
            const int o2 = o - kIq3TileSigns;
            const uint8_t *p = blk((o2 & 511) >> 3);
            if (p) v = iq3_signs(iq3_ld32(p + fo.words + 8 * (o2 >> 9) + (o2 & 7)));
        } else if (o < kIq3TileD) {         // [G][row] scales of words 2G, 2G+1, four rows
            const int o2 = o - kIq3TileScales;
            const int g = o2 >> 6;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint8_t *p = blk((o2 & 63) + i);
                if (p) {
                    const uint32_t s0 = iq3_ld32(p + fo.words + 8 * g) >> 28;
                    const uint32_t s1 = iq3_ld32(p + fo.words + 8 * g + 4) >> 28;
                    v |= (s0 | (s1 << 4)) << (8 * i);
                }
            }
        } else {                            // [row][2] d, two rows
            const int rr = (o - kIq3TileD) >> 1;
            const uint8_t *p0 = blk(rr);
            const uint8_t *p1 = blk(rr + 1);
            if (p0) v = *(const uint16_t *)(p0 + fo.d);
            if (p1) v |= (uint32_t)*(const uint16_t *)(p1 + fo.d) << 16;
        }
        out[u] = v;
    }
}

// Variant table: (waves, ring stages).
#define QWG_IQ3_VARIANTS(X) X(4, 2) X(4, 3) X(4, 4) X(8, 2) X(8, 3) X(16, 2) X(16, 3)

constexpr int iq3_key(int w, int r) { return w * 10 + r; }

}  // namespace

hipError_t launch_iq3_dequant(const uint8_t *src, const float *grid, float *dst,
                              int64_t nblocks, bool xxs, hipStream_t s) {
    int64_t groups = (nblocks + 3) / 4;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(iq3_dequant_kernel, dim3((unsigned)groups), dim3(256), 0, s, src, grid,
                       dst, nblocks, xxs);
    return hipGetLastError();
}

hipError_t launch_iq3_pack_tiles(const uint8_t *src, uint8_t *dst, int nb, int n_out, bool xxs,
                                 hipStream_t s) {
    const int64_t tiles = ((int64_t)n_out + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL(iq3_pack_tiles_kernel, dim3((unsigned)(tiles * nb)), dim3(256), 0, s, src,
                       dst, nb, n_out, xxs);
    return hipGetLastError();
}

bool iq3_rows_fits(int nb) { return nb <= kIq3RgMaxBlocks; }

hipError_t launch_iq3_rows(const GemvArgs &a, const float *grid, hipStream_t s) {
    if (a.nb > kIq3RgMaxBlocks) return hipErrorInvalidValue;
    const dim3 g((a.n_out + kIq3RgRows - 1) / kIq3RgRows);
    if (a.nb <= 8)
        hipLaunchKernelGGL((iq3_rows_kernel<1>), g, dim3(256), iq3_rg_lds(a.nb, 4), s, a, grid);
    else if (a.nb <= 16)
        hipLaunchKernelGGL((iq3_rows_kernel<2>), g, dim3(512), iq3_rg_lds(a.nb, 8), s, a, grid);
    else
        hipLaunchKernelGGL((iq3_rows_kernel<3>), g, dim3(768), iq3_rg_lds(a.nb, 12), s, a, grid);
    return hipGetLastError();
}

hipError_t launch_iq3_short(const GemvArgs &a, const ShortState &st, const float *grid,
                            hipStream_t s) {
    const bool tl = a.layout == kLayoutTiles;
    const int cols = (a.nb + a.splits - 1) / a.splits;
    const dim3 grid_dim(short_grid(a.tiles, a.splits));
    if (cols == 1)
        hipLaunchKernelGGL((iq3_short_kernel<1>), grid_dim, dim3(256), iq3_short_lds(1, tl), s, a, st, grid);
    else if (cols == 2)
        hipLaunchKernelGGL((iq3_short_kernel<2>), grid_dim, dim3(512), iq3_short_lds(2, tl), s, a, st, grid);
    else
        hipLaunchKernelGGL((iq3_short_kernel<4>), grid_dim, dim3(1024), iq3_short_lds(4, tl), s, a, st, grid);
    return hipGetLastError();
}

int iq3_stream_slots(const Iq3Shape &sh, bool tiled) {
    switch (iq3_key(sh.waves, sh.ring)) {
#define X(w, r) \
    case iq3_key(w, r): return tiled ? iq3_slots<w, r, true>() : iq3_slots<w, r, false>();
        QWG_IQ3_VARIANTS(X)
#undef X
        default: return 0;
    }
}

hipError_t launch_iq3_stream(const GroupArgs &g, const GemvArgs &single, const float *grid,
                             int nitems, const Iq3Shape &sh, bool tiled, hipStream_t s) {
    switch (iq3_key(sh.waves, sh.ring)) {
#define X(w, r) \
    case iq3_key(w, r): return iq3_launch<w, r>(g, single, grid, nitems, tiled, s);
        QWG_IQ3_VARIANTS(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qwg
