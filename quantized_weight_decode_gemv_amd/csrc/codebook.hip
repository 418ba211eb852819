// Codebook formats of the codebook.py page beyond IQ3_XXS (its format table,
// get_s, eff_np, dequant, and the IQ3_S branch of encode):
//   IQ3_S  110-byte blocks: fp16 d (bytes 0-1), 64 nine-bit grid indices (low
//          bytes at 2-65, ninth bits packed little-endian at 66-73), one sign
//          bit per weight (74-105), 4-bit sub-scales as nibbles (106-109);
//          eff = d*(1+2s), weight = +-grid[idx][t%4] * eff; grid [512][4].
//   IQ4_XS 136-byte blocks: fp16 d (0-1), 6-bit sub-scales (top two bits at
//          bits 2ib of the uint16 at 2-3, low four as nibbles at 4-7), 4-bit
//          codes at 8-135 (byte 8+16ib+j: weight j in the low nibble, weight
//          j+16 in the high one); eff = d*(s-32), weight = table[q] * eff.
// Dequantization is bit-exact. The GEMV runs on row-major blocks as a file
// stores them, or on a tile layout (each 64-row block column regrouped by
// field, as for IQ3), with a stream engine of 4-wavefront workgroups whose
// decode table (fp16) lives in LDS.
#include <cstdlib>

#include "qwg_device.h"

namespace qwg {

namespace {

__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) { return *(const uint16_t *)p; }

// ------------------------------------------------------------------ dequant

// One wavefront per block; lane l produces weights 4l..4l+3 (grid index l).
__global__ __launch_bounds__(256) void iq3s_dequant_kernel(const uint8_t *__restrict__ src,
                                                           const float *__restrict__ grid,
                                                           float *__restrict__ dst,
                                                           int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int ib = lane >> 3;
    for (int64_t blk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
         blk < nblocks; blk += nwaves) {
        const uint8_t *b = src + blk * kIq3sBytes;
        const float d = h2f_lo(ld_u16(b));
        const uint32_t idx = (uint32_t)b[2 + lane] | (((uint32_t)b[66 + (lane >> 3)] >> (lane & 7)) & 1u) << 8;
        const uint32_t sg = ((uint32_t)b[74 + (lane >> 1)] >> (4 * (lane & 1))) & 15u;
        const uint32_t s = ((uint32_t)b[106 + (ib >> 1)] >> (4 * (ib & 1))) & 15u;
        const float eff = __fmul_rn(d, __fadd_rn(1.0f, __fmul_rn(2.0f, (float)s)));
        const float4 g = *(const float4 *)(grid + 4 * idx);
        float4 o;
        o.x = __fmul_rn((sg & 1u) ? -g.x : g.x, eff);
        o.y = __fmul_rn((sg & 2u) ? -g.y : g.y, eff);
        o.z = __fmul_rn((sg & 4u) ? -g.z : g.z, eff);
        o.w = __fmul_rn((sg & 8u) ? -g.w : g.w, eff);
        // written once: non-temporal, as the Q4_K dequant's stores
        __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, (f32x4 *)(dst + blk * kQK + 4 * lane));
    }
}

// One wavefront per block; lane l produces weights 4m..4m+3 of sub-block l/8
// (m = l%8): low nibbles of code bytes 4m.. for m < 4, high nibbles of bytes
// 4(m-4).. otherwise. Blocks are 8-byte multiples, so with a 4-byte aligned
// source every code dword is aligned.
__global__ __launch_bounds__(256) void iq4xs_dequant_kernel(const uint8_t *__restrict__ src,
                                                            const float *__restrict__ table,
                                                            float *__restrict__ dst,
                                                            int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int ib = lane >> 3, m = lane & 7;
    // lane i holds value i % 16 of the table: a lookup is one cross-lane read
    // instead of a second memory round trip after the code word
    const float tv = table[lane & 15];
    for (int64_t blk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
         blk < nblocks; blk += nwaves) {
        const uint8_t *b = src + blk * kIq4xsBytes;
        const float d = h2f_lo(ld_u16(b));
        const uint32_t hi = ld_u16(b + 2);
        const uint32_t lo = ((uint32_t)b[4 + (ib >> 1)] >> (4 * (ib & 1))) & 15u;
        const uint32_t s = lo | ((hi >> (2 * ib)) & 3u) << 4;
        const float eff = __fmul_rn(d, __fsub_rn((float)s, 32.0f));
        const uint32_t word = *(const uint32_t *)(b + 8 + 16 * ib + 4 * (m & 3));
        const uint32_t sh = m >= 4 ? 4u : 0u;
        float4 o;
        o.x = __fmul_rn(__shfl(tv, (int)((word >> sh) & 15u)), eff);
        o.y = __fmul_rn(__shfl(tv, (int)((word >> (8 + sh)) & 15u)), eff);
        o.z = __fmul_rn(__shfl(tv, (int)((word >> (16 + sh)) & 15u)), eff);
        o.w = __fmul_rn(__shfl(tv, (int)((word >> (24 + sh)) & 15u)), eff);
        __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, (f32x4 *)(dst + blk * kQK + 32 * ib + 4 * m));
    }
}

// ------------------------------------------------------------------ tile layouts
//
// Column (t, b) of a tile-layout matrix (64 rows of block b) starts at
// (t*nb + b) * kCol; rows past n_out are zero blocks. Within a column the
// fields are grouped so that wavefront G (sub-blocks 2G and 2G+1) reads its
// row's pieces with aligned, conflict-free LDS reads.

// IQ3_S, 7040 bytes: indices [G][row][16] (bytes 2+16G..), signs [G][row][8]
// (74+8G..), ninth bits [G][row][2] (66+2G..), sub-scale bytes [row][4]
// (106..109), d [row][2] (0..1).
struct Iq3sFmt {
    // 4-wavefront workgroups, five per CU beside the 16 KB table. Measured on
    // the IQ3_S stream (us): 4 x 2 119.1, 4 x 3 125.7, 8 x 2 124.9, 16 x 2 162
    // (the 64 KB four-sign table, one 16-wavefront workgroup per CU: 127.0);
    // an SGPR cap changes nothing at this occupancy. Launches too short to
    // fill the chip without splitting their sums run 8 x 2 (two super-blocks
    // per stage): single GEMVs 5632 x 2048 / 2048 x 5632, tile layout, 11.4 /
    // 14.8 us with 4 x 2, 9.7 / 10.3 us with 8 x 2 (row-major 12.9 / 15.9 ->
    // 10.3 / 11.6 us).
    static constexpr int kShape = 42;         // 10 * wavefronts + ring stages
    static constexpr int kShapeSplit = 82;    // launches that split their sums
    static constexpr int kTable = 16384;      // decode table bytes at LDS address 0
    static constexpr bool kCapSgprs = false;  // stream kernel without an SGPR cap
    static constexpr int kBytes = kIq3sBytes;
    static constexpr int kCol = kTileRows * kIq3sBytes;
    static constexpr int kIdx = 0, kSign = 4096, kHb = 6144, kScale = 6656, kD = 6912;

    // Source byte of column byte o (even) and its row.
    __device__ static void source(int o, int &row, int &sbyte) {
        if (o < kSign) {
            row = (o >> 4) & 63;
            sbyte = 2 + 16 * (o >> 10) + (o & 15);
        } else if (o < kHb) {
            const int p = o - kSign;
            row = (p >> 3) & 63;
            sbyte = 74 + 8 * (p >> 9) + (p & 7);
        } else if (o < kScale) {
            const int p = o - kHb;
            row = (p >> 1) & 63;
            sbyte = 66 + 2 * (p >> 7);
        } else if (o < kD) {
            const int p = o - kScale;
            row = p >> 2;
            sbyte = 106 + (p & 3);
        } else {
            row = (o - kD) >> 1;
            sbyte = 0;
        }
    }

    // Half-group table at LDS address 0, 4 bytes per entry: entry
    // e = (s2 << 10) | (p << 9) | i holds components 2p and 2p+1 of grid row i
    // (nine bits) in fp16, each negated when its bit of s2 is set. 4096
    // entries, 16 KB (folding all four signs of a group into 8-byte entries
    // took 64 KB and left room for one workgroup per CU).
    // Returns false if a grid value this thread stored is not exactly fp16.
    // Each (p, i) pair's two fp16 magnitudes are converted once and its four
    // sign patterns made by flipping sign bits (conversion to fp16 rounds
    // symmetrically, so this is the fp16 of each signed value).
    __device__ static bool build_table(const float *grid, int t, int nthreads) {
        bool exact = true;
        for (int q = t; q < 1024; q += nthreads) {   // q = (p << 9) | i
            const float2 g = *(const float2 *)(grid + 4 * (q & 511) + 2 * (q >> 9));
            const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)g.x) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)g.y) << 16);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                *(__attribute__((address_space(3))) uint32_t *)(size_t)(((s2 << 10) | q) * 4) =
                    h ^ ((s2 & 1) ? 0x8000u : 0u) ^ ((s2 & 2) ? 0x80000000u : 0u);
            exact = exact && fp16_exact(g.x) && fp16_exact(g.y);
        }
        return exact;
    }

    // The bytes of one block that wavefront G uses: index bytes 2+16G..17+16G,
    // sign bytes 74+8G..81+8G, ninth-bit bytes 66+2G and 67+2G (low half),
    // sub-scale bytes 106..109 and d (low half).
    struct Raw {
        uint32_t q[4], sg[2], hb, sc, d16;
    };
    // Row windows (row-major weights): granules 0..7 of a 144-byte window hold
    // the block (it starts at an even window byte sh <= 14 and ends by 124).
    static constexpr int kWinGran = 8;

    // From a tile-layout column (this lane's row).
    template <int G>
    __device__ static void fetch_tiled(const uint8_t *col, int lane, Raw &r) {
        const uint4 q = *(const uint4 *)(col + kIdx + G * 1024 + 16 * lane);
        const uint2 sg = *(const uint2 *)(col + kSign + G * 512 + 8 * lane);
        r.q[0] = q.x;
        r.q[1] = q.y;
        r.q[2] = q.z;
        r.q[3] = q.w;
        r.sg[0] = sg.x;
        r.sg[1] = sg.y;
        r.hb = ld_u16(col + kHb + G * 128 + 2 * lane);
        r.sc = *(const uint32_t *)(col + kScale + 4 * lane);
        r.d16 = ld_u16(col + kD + 2 * lane);
    }

    // From a row window in LDS (16-byte aligned; the block starts at byte sh,
    // even). Every field starts 0 or 2 bytes into a dword: whole dwords are
    // read and realigned with v_alignbyte (the dword past a field is read only
    // to supply bytes that the shift drops when the offset is 0).
    template <int G>
    __device__ static void fetch_window(const uint8_t *win, uint32_t sh, Raw &r) {
        const uint32_t *p = (const uint32_t *)win;
        const uint32_t o = sh + 2u;                 // indices at block byte 2 + 16G
        const uint32_t sft = o & 3u;                // = (sh + 74) & 3 = (sh + 106) & 3
        const uint32_t qd = (o >> 2) + 4 * G;
        uint32_t a[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) a[i] = p[qd + i];
#pragma unroll
        for (int i = 0; i < 4; ++i) r.q[i] = __builtin_amdgcn_alignbyte(a[i + 1], a[i], sft);
        const uint32_t sd = ((sh + 74u) >> 2) + 2 * G;
        const uint32_t v0 = p[sd], v1 = p[sd + 1], v2 = p[sd + 2];
        r.sg[0] = __builtin_amdgcn_alignbyte(v1, v0, sft);
        r.sg[1] = __builtin_amdgcn_alignbyte(v2, v1, sft);
        const uint32_t oh = sh + 66u + 2 * G;
        r.hb = (p[oh >> 2] >> ((oh & 2u) << 3)) & 0xFFFFu;
        const uint32_t cd = (sh + 106u) >> 2;
        r.sc = __builtin_amdgcn_alignbyte(p[cd + 1], p[cd], sft);
        r.d16 = (p[sh >> 2] >> ((sh & 2u) << 3)) & 0xFFFFu;
    }

    // From global memory, 2 bytes at a time (the block is 2-byte aligned).
    template <int G>
    __device__ static void fetch_direct(const uint8_t *blk, Raw &r) {
        const uint16_t *h = (const uint16_t *)blk;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.q[i] = (uint32_t)h[1 + 8 * G + 2 * i] | ((uint32_t)h[2 + 8 * G + 2 * i] << 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            r.sg[i] = (uint32_t)h[37 + 4 * G + 2 * i] | ((uint32_t)h[38 + 4 * G + 2 * i] << 16);
        r.hb = h[33 + G];
        r.sc = (uint32_t)h[53] | ((uint32_t)h[54] << 16);
        r.d16 = h[0];
    }

    // Eight rows rit..rit+7 (rit a multiple of 8) of a tile-layout column as
    // 55 granules: index runs [G][8][16], sign runs [G][8][8], ninth-bit runs
    // [G][8][2], sub-scales [8][4], d [8][2] (880 bytes); the byte offset in
    // the column of granule g, and the fields of slice row r.
    static constexpr int kSliceGran = 55;
    __device__ static int slice_off(int g, int rit) {
        if (g < 32) return kIdx + (g >> 3) * 1024 + 16 * rit + 16 * (g & 7);
        if (g < 48) return kSign + ((g - 32) >> 2) * 512 + 8 * rit + 16 * ((g - 32) & 3);
        if (g < 52) return kHb + (g - 48) * 128 + 2 * rit;
        if (g < 54) return kScale + 4 * rit + 16 * (g - 52);
        return kD + 2 * rit;
    }
    template <int G>
    __device__ static void fetch_slice(const uint8_t *sl, int r, Raw &raw) {
        const uint4 q = *(const uint4 *)(sl + G * 128 + 16 * r);
        const uint2 sg = *(const uint2 *)(sl + 512 + G * 64 + 8 * r);
        raw.q[0] = q.x;
        raw.q[1] = q.y;
        raw.q[2] = q.z;
        raw.q[3] = q.w;
        raw.sg[0] = sg.x;
        raw.sg[1] = sg.y;
        raw.hb = ld_u16(sl + 768 + G * 16 + 2 * r);
        raw.sc = *(const uint32_t *)(sl + 832 + 4 * r);
        raw.d16 = ld_u16(sl + 864 + 2 * r);
    }

    // acc + this lane's row sum over wavefront G's 64 weights. Group k (four
    // weights) of sub-block h reads two entries, halves p = 0 and 1: ((two
    // sign bits of nibble k) << 10 | p << 9 | ninth bit << 8 | index byte),
    // each assembled by one v_perm from the index dword and a dword of bytes
    // (s2 << 2 | p << 1 | ninth bit) built once per sub-block.
    // (xat(i): activation i of the wavefront's 64: scalar loads in the
    // stream, registers in the row-group kernel)
    template <int G, typename XAt>
    __device__ static float dot(const Raw &r, int, XAt xat, float acc) {
        const uint2 sg = {r.sg[0], r.sg[1]};
        const uint32_t hb = r.hb, sc = r.sc;
        const float d = h2f_lo(r.d16);
        const uint32_t idx[4] = {r.q[0], r.q[1], r.q[2], r.q[3]};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t S = h ? sg.y : sg.x;
            // byte b of S holds sign nibbles 2b (bits 0-3) and 2b+1 (bits 4-7);
            // bring each pair of sign bits to bits 2-3 of a byte
            const uint32_t le = (S << 2) & 0x0C0C0C0Cu;   // nibbles 0, 2, 4, 6: bits 0-1
            const uint32_t lo = (S >> 2) & 0x0C0C0C0Cu;   // nibbles 1, 3, 5, 7: bits 0-1
            const uint32_t he = S & 0x0C0C0C0Cu;          // nibbles 0, 2, 4, 6: bits 2-3
            const uint32_t ho = (S >> 4) & 0x0C0C0C0Cu;   // nibbles 1, 3, 5, 7: bits 2-3
            const uint32_t H = hb >> (8 * h);
            const uint32_t n03 = ((H & 15u) * 0x00204081u) & 0x01010101u;
            const uint32_t n47 = (((H >> 4) & 15u) * 0x00204081u) & 0x01010101u;
            const uint32_t ca0 = __builtin_amdgcn_perm(lo, le, 0x05010400u) | n03;
            const uint32_t cb0 = __builtin_amdgcn_perm(lo, le, 0x07030602u) | n47;
            const uint32_t ca1 = __builtin_amdgcn_perm(ho, he, 0x05010400u) | n03 | 0x02020202u;
            const uint32_t cb1 = __builtin_amdgcn_perm(ho, he, 0x07030602u) | n47 | 0x02020202u;
            const uint32_t s = (sc >> (8 * G + 4 * h)) & 15u;
            const float eff = d * (1.0f + 2.0f * (float)s);
            auto x = [&](int i) { return xat(32 * h + i); };
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t sel = (uint32_t)(k & 3) | ((uint32_t)(4 + (k & 3)) << 8) | 0x0C0C0000u;
                const uint32_t iw = idx[2 * h + (k >> 2)];
                const uint32_t t0 = __builtin_amdgcn_perm(k < 4 ? ca0 : cb0, iw, sel);
                const uint32_t t1 = __builtin_amdgcn_perm(k < 4 ? ca1 : cb1, iw, sel);
                const uint32_t v0 = lds_load<uint32_t>(t0 << 2);
                const uint32_t v1 = lds_load<uint32_t>(t1 << 2);
                s0 = __builtin_fmaf(h2f_lo(v0), x(4 * k + 0), s0);
                s1 = __builtin_fmaf(h2f_hi(v0), x(4 * k + 1), s1);
                s0 = __builtin_fmaf(h2f_lo(v1), x(4 * k + 2), s0);
                s1 = __builtin_fmaf(h2f_hi(v1), x(4 * k + 3), s1);
            }
            acc = __builtin_fmaf(eff, s0 + s1, acc);
        }
        return acc;
    }
};

// IQ4_XS, 8704 bytes: codes [G][row][32] (bytes 8+32G..), header [row][8]
// (bytes 0..7: d, the scales' top bits, their low nibbles).
struct Iq4xsFmt {
    // 4-wavefront workgroups, seven per CU (LDS 22.5 KB each), SGPRs capped so
    // that the register file allows them. Measured on the IQ4_XS stream (us):
    // 4 x 2 capped 109-112, uncapped 115; 8 x 2 119; 16 x 2 151; the 64 KB pair
    // table this replaced, one 16-wavefront workgroup per CU: 121. Split
    // launches 8 x 2: single GEMVs (tile layout) 10.7 / 12.4 us -> 9.7 / 9.7 us.
    static constexpr int kShape = 42;
    static constexpr int kShapeSplit = 82;
    static constexpr int kTable = 4096;
    static constexpr bool kCapSgprs = true;   // 96 SGPRs: eight wavefronts per SIMD
    static constexpr int kBytes = kIq4xsBytes;
    static constexpr int kCol = kTileRows * kIq4xsBytes;
    static constexpr int kCodes = 0, kHead = 8192;

    __device__ static void source(int o, int &row, int &sbyte) {
        if (o < kHead) {
            row = (o >> 5) & 63;
            sbyte = 8 + 32 * (o >> 11) + (o & 31);
        } else {
            row = (o - kHead) >> 3;
            sbyte = (o - kHead) & 7;
        }
    }

    // Table at LDS address 0, one copy per lane: entry (code v, lane c) at
    // v*256 + 4c holds table[v] in fp16 in both halves, so the 64 lanes of a
    // read always hit 64 different banks. 4 KB (a pair table indexed by the
    // whole code byte took 64 KB and left room for one workgroup per CU).
    // Returns false if a table value this thread stored is not exactly fp16.
    __device__ static bool build_table(const float *table, int t, int nthreads) {
        bool exact = true;
        for (int e = t; e < 1024; e += nthreads) {
            const float v = table[e >> 6];
            const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)v);
            *(__attribute__((address_space(3))) uint32_t *)(size_t)(e * 4) = h | (h << 16);
            exact = exact && fp16_exact(v);
        }
        return exact;
    }

    // The bytes of one block that wavefront G uses: code bytes 8+32G..39+32G
    // and header bytes 0..7.
    struct Raw {
        uint32_t q[8];
        uint2 hd;
    };
    // Row windows (row-major weights): the block starts at window byte 0 or 8
    // (the weights 16-byte aligned, blocks 8 bytes apart) and takes all nine
    // granules of the 144-byte window.
    static constexpr int kWinGran = 9;

    template <int G>
    __device__ static void fetch_tiled(const uint8_t *col, int lane, Raw &r) {
        const uint4 qa = *(const uint4 *)(col + kCodes + G * 2048 + 32 * lane);
        const uint4 qb = *(const uint4 *)(col + kCodes + G * 2048 + 32 * lane + 16);
        r.q[0] = qa.x;
        r.q[1] = qa.y;
        r.q[2] = qa.z;
        r.q[3] = qa.w;
        r.q[4] = qb.x;
        r.q[5] = qb.y;
        r.q[6] = qb.z;
        r.q[7] = qb.w;
        r.hd = *(const uint2 *)(col + kHead + 8 * lane);
    }

    // From a row window in LDS (sh = 0 or 8: every field 8-byte aligned).
    template <int G>
    __device__ static void fetch_window(const uint8_t *win, uint32_t sh, Raw &r) {
        const u32x2 *p = (const u32x2 *)(win + sh + 8 + 32 * G);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x2 v = p[i];
            r.q[2 * i] = v.x;
            r.q[2 * i + 1] = v.y;
        }
        const u32x2 h = *(const u32x2 *)(win + sh);
        r.hd = make_uint2(h.x, h.y);
    }

    // From global memory (the block is 8-byte aligned).
    template <int G>
    __device__ static void fetch_direct(const uint8_t *blk, Raw &r) {
        const uint2 *p = (const uint2 *)(blk + 8 + 32 * G);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint2 v = p[i];
            r.q[2 * i] = v.x;
            r.q[2 * i + 1] = v.y;
        }
        r.hd = *(const uint2 *)blk;
    }

    // Eight rows rit..rit+7 of a tile-layout column as 68 granules: code runs
    // [G][8][32], then bytes 0-7 [8][8] (1088 bytes).
    static constexpr int kSliceGran = 68;
    __device__ static int slice_off(int g, int rit) {
        if (g < 64) return kCodes + (g >> 4) * 2048 + 32 * rit + 16 * (g & 15);
        return kHead + 8 * rit + 16 * (g - 64);
    }
    template <int G>
    __device__ static void fetch_slice(const uint8_t *sl, int r, Raw &raw) {
        const uint4 qa = *(const uint4 *)(sl + G * 256 + 32 * r);
        const uint4 qb = *(const uint4 *)(sl + G * 256 + 32 * r + 16);
        raw.q[0] = qa.x;
        raw.q[1] = qa.y;
        raw.q[2] = qa.z;
        raw.q[3] = qa.w;
        raw.q[4] = qb.x;
        raw.q[5] = qb.y;
        raw.q[6] = qb.z;
        raw.q[7] = qb.w;
        raw.hd = *(const uint2 *)(sl + 1024 + 8 * r);
    }

    // Byte j of sub-block h's sixteen code bytes gives weights j (low nibble)
    // and j + 16 (high nibble). The nibbles of four bytes are split into bytes
    // with two masks; then per weight one v_perm forms v*256 + 4*lane and one
    // LDS read returns the table value.
    template <int G, typename XAt>
    __device__ static float dot(const Raw &r, int lane, XAt xat, float acc) {
        const uint2 hd = r.hd;
        const uint4 qa = {r.q[0], r.q[1], r.q[2], r.q[3]};
        const uint4 qb = {r.q[4], r.q[5], r.q[6], r.q[7]};
        const float d = h2f_lo(hd.x);
        const uint32_t sh = hd.x >> 16;
        const uint32_t lofs = (uint32_t)lane * 4u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            constexpr int kIb0 = 2 * G;
            const int ib = kIb0 + h;
            const uint32_t s = ((hd.y >> (4 * ib)) & 15u) | (((sh >> (2 * ib)) & 3u) << 4);
            const float eff = d * ((float)s - 32.0f);
            const uint32_t Q[4] = {h ? qb.x : qa.x, h ? qb.y : qa.y, h ? qb.z : qa.z,
                                   h ? qb.w : qa.w};
            auto x = [&](int i) { return xat(32 * h + i); };
            float s0 = 0.0f, s1 = 0.0f;
            // The 16 table reads of two code words and their 16 activations are
            // issued before the FMAs (LDS and scalar loads share one wait
            // counter; interleaved, each pair waited out a round trip).
            // Measured: IQ4_XS stream 111.1 -> 108.5-109.5 us.
#pragma unroll
            for (int qq = 0; qq < 4; qq += 2) {
                uint32_t va[8], vb[8];
#pragma unroll
                for (int q = qq; q < qq + 2; ++q) {
                    const uint32_t lo = Q[q] & 0x0F0F0F0Fu;
                    const uint32_t hi = (Q[q] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t sel = 0x0C0C0004u | ((uint32_t)k << 8);
                        va[4 * (q - qq) + k] = lds_load<uint32_t>(__builtin_amdgcn_perm(lofs, lo, sel));
                        vb[4 * (q - qq) + k] = lds_load<uint32_t>(__builtin_amdgcn_perm(lofs, hi, sel));
                    }
                }
                float xa[8], xb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    xa[i] = x(4 * qq + i);
                    xb[i] = x(16 + 4 * qq + i);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    s0 = __builtin_fmaf(h2f_lo(va[i]), xa[i], s0);
                    s1 = __builtin_fmaf(h2f_lo(vb[i]), xb[i], s1);
                }
            }
            acc = __builtin_fmaf(eff, s0 + s1, acc);
        }
        return acc;
    }
};

// Row-major blocks -> tile layout, one workgroup per (tile, block column), in
// 2-byte units (IQ3_S blocks are only 2-byte aligned).
template <class F>
__global__ __launch_bounds__(256) void cb_pack_tiles_kernel(const uint8_t *__restrict__ src,
                                                            uint8_t *__restrict__ dst, int nb,
                                                            int n_out) {
    const int b = blockIdx.x % nb;
    const int tile = blockIdx.x / nb;
    const int64_t row_bytes = (int64_t)nb * F::kBytes;
    uint16_t *out = (uint16_t *)(dst + (int64_t)blockIdx.x * F::kCol);
    for (int u = threadIdx.x; u < F::kCol / 2; u += blockDim.x) {
        int rr, sbyte;
        F::source(2 * u, rr, sbyte);
        const int r = tile * kTileRows + rr;
        uint16_t v = 0;
        if (r < n_out)
            v = *(const uint16_t *)(src + r * row_bytes + (int64_t)b * F::kBytes + sbyte);
        out[u] = v;
    }
}

// ------------------------------------------------------------------ stream engine
//
// As the IQ3 engine: persistent workgroups walk work items (64-row tile x
// super-block range); wavefront 4j + G computes sub-blocks 2G, 2G+1 of
// super-block j of each stage for the 64 rows (lane = row), with the
// activations as scalar operands; an R-slot ring filled by LDS-DMA runs ahead
// across items. The decode table sits at LDS address 0 (IQ3_S 16 KB, IQ4_XS
// 4 KB), small enough for five or seven 4-wavefront workgroups per CU.
//
// Two weight layouts (TL): the tile layout, whose stage columns are copied
// whole; and row-major blocks as a file stores them, where each stage copies
// for every row the 16-byte granules that hold its block into a 144-byte row
// window (nine granules: 36 dwords apart, so the 64 lanes' reads spread over
// the banks). The weights must then start on a 16-byte boundary (so no block
// starts before it); a granule past the buffer's end is clamped to the last
// whole one inside, and the one block that such a granule can hold (the last
// row's last block, when the buffer ends off a boundary) is read directly
// from memory by its lane.
template <class F, int W, int R, bool TL>
struct CbCfg {
    static constexpr int kBps = W / 4;
    static constexpr int kWin = 144;                              // row window bytes
    static constexpr int kCol = TL ? F::kCol : kTileRows * kWin;  // one block column in LDS
    static constexpr int kGran = kCol / 16;                       // 16-byte granules per column
    static constexpr int kTable = F::kTable;                      // at LDS address 0
    static constexpr int kRing = kTable;
    static constexpr int kSlot = kBps * kCol;
    static constexpr int kRed = kRing + R * kSlot;    // [W][64] fp32 row sums
    static constexpr int kLds = kRed + W * 64 * 4;
    static_assert(kCol % 16 == 0, "columns are whole granules");
    static_assert(kGran <= 3 * 256, "a column takes at most three copy rounds");
    // copy instructions per stage of wavefront G: rounds i with 256i + 64G < kGran
    // (in a row window some lanes of a round may idle, never all of them)
    static constexpr int copies(int G) {
        return (64 * G < kGran) + (256 + 64 * G < kGran) + (512 + 64 * G < kGran);
    }
};

struct CbItem {
    GemvArgs a;
    const uint8_t *sb;   // tile layout: the tile's column 0; rows: its first row, rounded down to 16 bytes
    uint32_t sb_off;     // rows: that row's offset from sb (0..15)
    uint32_t hi;         // rows: last 16-byte granule wholly inside the weights, relative to sb (capped)
    int tile, split, kb0, kb1, nst, row0;
    bool tail;           // rows: holds the last row's last block and the buffer ends off a granule
};

template <class F, int BPS, bool TL>
__device__ __forceinline__ void cb_load_item(CbItem &it, int k, const GroupArgs &g,
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
    it.tile = local / splits;
    it.split = local - it.tile * splits;
    it.kb0 = it.split * it.a.nb / splits;
    it.kb1 = (it.split + 1) * it.a.nb / splits;
    it.nst = (it.kb1 - it.kb0 + BPS - 1) / BPS;
    it.row0 = it.tile * kTileRows;
    if constexpr (TL) {
        it.sb = it.a.w + (int64_t)it.tile * it.a.nb * F::kCol;
        it.sb_off = 0;
        it.hi = 0;
        it.tail = false;
        return;
    }
    const uintptr_t wb = (uintptr_t)it.a.w;   // 16-byte aligned
    const uintptr_t we = wb + (uintptr_t)it.a.n_out * (uintptr_t)it.a.row_bytes;
    const uintptr_t base0 = wb + (uintptr_t)it.row0 * (uintptr_t)it.a.row_bytes;
    const uintptr_t sb = base0 & ~(uintptr_t)15;
    it.sb = (const uint8_t *)sb;
    it.sb_off = (uint32_t)(base0 & 15);
    // The tile's first row starts at least one block (>= 110 bytes) before the
    // end, so the last whole granule lies at or after sb.
    const uintptr_t hi16 = (we & ~(uintptr_t)15) - 16;
    it.hi = hi16 - sb < 0x40000000u ? (uint32_t)(hi16 - sb) : 0x40000000u;
    it.tail = (we & 15) != 0 && it.row0 + kTileRows >= it.a.n_out && it.kb1 == it.a.nb;
}

template <class F, int G, int W, int R, bool TL>
__device__ __forceinline__ void cb_stream(const GroupArgs &g, const GemvArgs &single,
                                          const float *tab, int nitems, uint8_t *smem) {
    static_assert(R >= 2 && R <= 4, "ring of two to four stages");
    using C = CbCfg<F, W, R, TL>;
    constexpr int BPS = C::kBps;
    constexpr int kCp = C::copies(G);
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const int wave = 4 * j + G;
    const int stride = gridDim.x;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    int kc = skip_holes(blockIdx.x, stride, nitems, g);
    if (kc >= nitems) return;
    CbItem c;
    cb_load_item<F, BPS, TL>(c, kc, g, single);

    // Row windows: round i of this wavefront copies granule k = 256i + 64G + lane
    // of the column, granule k % 9 of row k / 9's window (LDS byte 16k).
    int crow[3];
    uint32_t cgran[3];
    bool cact[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int k = 256 * i + 64 * G + lane;
        crow[i] = min(k / 9, kTileRows - 1);
        cgran[i] = 16u * (uint32_t)(k % 9);
        cact[i] = k < C::kGran && k % 9 < F::kWinGran;
    }

    int kd = kc, sd = 0, slot_d = 0, pending = 0;
    CbItem d = c;
    uint32_t doff[3];  // rows: this lane's granule of block 0 of its row, relative to d.sb
    auto prep_copy = [&]() {
        if constexpr (TL) return;
#pragma unroll
        for (int i = 0; i < 3; ++i)
            doff[i] = d.sb_off +
                      (uint32_t)(min(d.row0 + crow[i], d.a.n_out - 1) - d.row0) *
                          (uint32_t)d.a.row_bytes +
                      cgran[i];
    };
    prep_copy();
    uint32_t flags = 0;  // bit k: this wavefront's copies are in ring slot k
    auto issue_next = [&]() {
        if (kd >= nitems) return;
        const int b = d.kb0 + sd * BPS + j;
        if (b < d.kb1) {
            const uint32_t colb = lds0 + C::kRing + slot_d * C::kSlot + j * C::kCol;
            if constexpr (TL) {
                const uint8_t *src = d.sb + (int64_t)b * F::kCol;
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int g0 = 256 * i + 64 * G;    // this wavefront's first granule of round i
                    if (g0 < C::kGran) {
                        if (g0 + lane < C::kGran)
                            dma16_stream(src + 16 * (g0 + lane), colb + 16 * g0);
                    }
                }
            } else {
                const uint32_t boff = (uint32_t)(F::kBytes * b);
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int g0 = 256 * i + 64 * G;
                    if (g0 < C::kGran) {
                        if (cact[i]) {
                            // (offset + a multiple of 16) & ~15 keeps the granule index
                            const uint32_t off = min((doff[i] + boff) & ~15u, d.hi);
                            dma16(d.sb, off, colb + 16 * g0);
                        }
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
                cb_load_item<F, BPS, TL>(d, kd, g, single);
                prep_copy();
            }
        }
    };
#pragma unroll
    for (int i = 0; i < R - 1; ++i) issue_next();

    // The decode table, while the first stages are in flight. A value that
    // fp16 cannot hold would be rounded in it: the workgroup then stores NaN in
    // every row instead (host code that creates a group rejects such a table
    // up front). The vote goes through a word of the row-sum buffer, idle
    // until the first item ends.
    volatile uint32_t *vote = (volatile uint32_t *)(smem + C::kRed);
    if (threadIdx.x == 0) *vote = 0u;
    lds_barrier();
    const bool exact = F::build_table(tab, (int)threadIdx.x, W * 64);
    if (__builtin_amdgcn_ballot_w64(!exact) != 0 && lane == 0) *vote = 1u;
    lds_barrier();
    const bool grid_bad = __builtin_amdgcn_readfirstlane(*vote) != 0u;

    float *red = (float *)(smem + C::kRed);
    int slot_c = 0;
    for (;;) {
        const int row = c.row0 + lane;
        // rows: low bits of this lane's row address (block offsets within granules)
        const uint32_t rlo = (uint32_t)(uintptr_t)c.a.w +
                             (uint32_t)min(row, c.a.n_out - 1) * (uint32_t)c.a.row_bytes;
        float acc = 0.0f;
        for (int s = 0; s < c.nst; ++s) {
            const int nxt = slot_c + 1 == R ? 0 : slot_c + 1;
            // copies of the stages after this one may stay in flight
            int younger = 0;
            if (R >= 3 && pending > 1) younger += kCp * (int)((flags >> nxt) & 1u);
            if (R >= 4 && pending > 2)
                younger += kCp * (int)((flags >> (nxt + 1 == R ? 0 : nxt + 1)) & 1u);
            wait_vmcnt_upto(younger);
            lds_barrier();   // stage in slot_c complete for every wavefront (and the table)
            issue_next();
            const int b = c.kb0 + s * BPS + j;
            if (b < c.kb1) {
                const uint8_t *col = smem + C::kRing + slot_c * C::kSlot + j * C::kCol;
                typename F::Raw raw;
                if constexpr (TL) {
                    F::template fetch_tiled<G>(col, lane, raw);
                } else {
                    const uint32_t sh = (rlo + (uint32_t)(F::kBytes * b)) & 15u;
                    F::template fetch_window<G>(col + C::kWin * lane, sh, raw);
                    if (c.tail && b == c.a.nb - 1) {   // wave-uniform, once per matrix
                        if (row == c.a.n_out - 1)
                            F::template fetch_direct<G>(
                                c.a.w + (int64_t)row * c.a.row_bytes + (int64_t)F::kBytes * b, raw);
                    }
                }
                const cfloat_p xg = as_scalar(c.a.x) + (int64_t)kQK * b + 64 * G;
                acc = F::template dot<G>(raw, lane, [&](int i) { return xg[i]; }, acc);
            }
            --pending;
            slot_c = nxt;
        }
        red[wave * 64 + lane] = acc;
        lds_barrier();
        if (wave == 0) {
            float tsum = red[lane];
            for (int w = 1; w < W; ++w) tsum += red[w * 64 + lane];
            if (grid_bad) tsum = __builtin_nanf("");
            const float total[1] = {tsum};
            tile_epilogue<1>(c.a, c.tile, c.split, total);
        }
        kc = skip_holes(kc + stride, stride, nitems, g);
        if (kc >= nitems) break;
        cb_load_item<F, BPS, TL>(c, kc, g, single);
    }
}

template <class F, int W, int R, bool TL>
__device__ __forceinline__ void cb_stream_entry(GroupArgs g, GemvArgs single, const float *tab,
                                                int nitems) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    switch (__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3)) {
        case 0: cb_stream<F, 0, W, R, TL>(g, single, tab, nitems, smem); break;
        case 1: cb_stream<F, 1, W, R, TL>(g, single, tab, nitems, smem); break;
        case 2: cb_stream<F, 2, W, R, TL>(g, single, tab, nitems, smem); break;
        default: cb_stream<F, 3, W, R, TL>(g, single, tab, nitems, smem); break;
    }
}

// The same kernel with and without an SGPR cap (the attribute takes no
// template argument); F::kCapSgprs picks one.
template <class F, int W, int R, bool TL>
__global__ __launch_bounds__(W * 64) void cb_stream_kernel(GroupArgs g, GemvArgs single,
                                                           const float *tab, int nitems) {
    cb_stream_entry<F, W, R, TL>(g, single, tab, nitems);
}

template <class F, int W, int R, bool TL>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_num_sgpr(96))) void cb_stream_kernel96(
    GroupArgs g, GemvArgs single, const float *tab, int nitems) {
    cb_stream_entry<F, W, R, TL>(g, single, tab, nitems);
}

template <class F, int W, int R, bool TL>
constexpr auto cb_kernel() {
    if constexpr (F::kCapSgprs)
        return cb_stream_kernel96<F, W, R, TL>;
    else
        return cb_stream_kernel<F, W, R, TL>;
}

// Engine shapes (wavefronts, ring stages). QWG_CB_SHAPE = 10*W + R picks one
// for both formats and layouts (tuning experiments).
#define QWG_CB_SHAPES(X) X(16, 2) X(16, 3) X(12, 3) X(8, 2) X(8, 3) X(8, 4) X(4, 2) X(4, 3)

template <class F, int W, int R, bool TL>
int cb_slots_wr() {
    // a function-local static: initialised once even under concurrent first calls
    static const int slots = [] {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        constexpr size_t lds = CbCfg<F, W, R, TL>::kLds;
        if (lds > 160 * 1024 ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cb_kernel<F, W, R, TL>(), W * 64,
                                                         lds) != hipSuccess ||
            per_cu < 1)
            per_cu = lds > 160 * 1024 ? 0 : 1;
        return per_cu * cus;
    }();
    return slots;
}

template <class F, int W, int R, bool TL>
hipError_t cb_launch_wr(const GroupArgs &g, const GemvArgs &single, const float *tab, int nitems,
                        hipStream_t s) {
    int n = cb_slots_wr<F, W, R, TL>();
    if (n <= 0) return hipErrorInvalidValue;
    if (n > nitems) n = nitems;
    constexpr size_t lds = CbCfg<F, W, R, TL>::kLds;
    hipLaunchKernelGGL((cb_kernel<F, W, R, TL>()), dim3((unsigned)n), dim3(W * 64), lds, s, g,
                       single, tab, nitems);
    return hipGetLastError();
}

template <class F, bool TL>
int cb_slots_any(int shape) {
    switch (shape) {
#define X(w, r) \
    case 10 * w + r: return cb_slots_wr<F, w, r, TL>();
        QWG_CB_SHAPES(X)
#undef X
        default: return 0;
    }
}

// QWG_CB_SHAPE = 10*W + R overrides the shape of every launch of both formats
// and layouts (tuning experiments); 0 if unset or not a valid shape.
template <class F>
int cb_env_shape() {
    static const int v = [] {
        const char *e = getenv("QWG_CB_SHAPE");
        const int k = e ? atoi(e) : 0;
        switch (k) {
#define X(w, r) case 10 * w + r:
            QWG_CB_SHAPES(X)
#undef X
            return cb_slots_any<F, true>(k) > 0 && cb_slots_any<F, false>(k) > 0 ? k : 0;
            default: return 0;
        }
    }();
    return v;
}

template <class F>
int cb_shape_f(bool split) {
    const int e = cb_env_shape<F>();
    return e ? e : split ? F::kShapeSplit : F::kShape;
}

template <class F, bool TL>
hipError_t cb_launch(int shape, const GroupArgs &g, const GemvArgs &single, const float *tab,
                     int nitems, hipStream_t s) {
    switch (shape) {
#define X(w, r) \
    case 10 * w + r: return cb_launch_wr<F, w, r, TL>(g, single, tab, nitems, s);
        QWG_CB_SHAPES(X)
#undef X
        default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------------ row groups
//
// Single GEMVs of at most 24 blocks per row on up to one 64-row tile per
// compute unit (the Q4_K and IQ3 row-group scheme): a workgroup of 4 NS
// wavefronts takes eight whole rows, so no split sums meet through memory.
// Wavefront w takes pair G = w % 4 of sub-blocks of the blocks of set w / 4,
// lane r + 8s row r's block s + 8 (w / 4), its 64 activations in registers.
// The table is built first (it reads the grid or table from global memory);
// row-major rows arrive as one contiguous run of 16-byte granules (w is
// 16-byte aligned; granules past the buffer's end are clamped and the last
// block, if it reaches into a clamped granule, is read directly), tile-layout
// rows as each column's eight-row slice.
constexpr int kCbRgRows = 8;
constexpr int kCbRgMaxBlocks = 24;
template <class F>
__host__ __device__ constexpr int cb_rg_region(int nb) {
    const int run = (15 + kCbRgRows * nb * F::kBytes + 15) / 16 + 1;
    const int gr = run > F::kSliceGran * nb ? run : F::kSliceGran * nb;
    return (gr + 63) / 64 * 64 * 16;
}
template <class F>
__host__ __device__ constexpr int cb_rg_lds(int nb, int waves) {
    return F::kTable + cb_rg_region<F>(nb) + waves * kCbRgRows * 4 + 64;
}
static_assert(cb_rg_lds<Iq3sFmt>(kCbRgMaxBlocks, 12) <= 65536, "LDS of one workgroup");
static_assert(cb_rg_lds<Iq4xsFmt>(kCbRgMaxBlocks, 12) <= 65536, "LDS of one workgroup");

template <class F, int G>
__device__ __forceinline__ float cb_rows_dot(const GemvArgs &a, const uint8_t *rg, uint32_t o,
                                             int row, int b, int r, int lane,
                                             const f32x4 (&xv)[16]) {
    typename F::Raw raw;
    if (a.layout == kLayoutTiles) {
        F::template fetch_slice<G>(rg + b * (kCbRgRows * F::kBytes), r, raw);
    } else {
        F::template fetch_window<G>(rg + (o & ~15u), o & 15u, raw);
        const uintptr_t we = (uintptr_t)a.w + (uintptr_t)a.n_out * (uintptr_t)a.row_bytes;
        if ((we & 15) != 0 && row == a.n_out - 1 && b == a.nb - 1)
            F::template fetch_direct<G>(a.w + (int64_t)row * a.row_bytes + F::kBytes * b, raw);
    }
    return F::template dot<G>(raw, lane, [&](int i) { return xv[i >> 2][i & 3]; }, 0.0f);
}

template <class F, int NS>
__global__ __launch_bounds__(256 * NS) void cb_rows_kernel(GemvArgs a, const float *tab) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int R = kCbRgRows;
    constexpr int W = 4 * NS;
    const bool tl = a.layout == kLayoutTiles;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = wave & 3;
    const int nb = a.nb;
    const int row0 = blockIdx.x * R;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t rgb = lds0 + F::kTable;
    const int r = lane & (R - 1);
    const int b = (lane >> 3) + 8 * (wave >> 2);

    f32x4 xv[16];
    {
        const f32x4 *xp = (const f32x4 *)(a.x + (int64_t)kQK * min(b, nb - 1) + 64 * G);
#pragma unroll
        for (int q = 0; q < 16; ++q) xv[q] = xp[q];
    }
    uint32_t o0 = 0;
    if (tl) {
        constexpr int GPB = F::kSliceGran;
        const int nk = GPB * nb;
        const int rit = row0 & 63;
        for (int k0 = 64 * wave; k0 < nk; k0 += 64 * W) {
            const int k = min(k0 + lane, nk - 1);
            const int bb = k / GPB;
            dma16(a.w + ((int64_t)(row0 >> 6) * nb + bb) * F::kCol + F::slice_off(k - GPB * bb, rit),
                  rgb + 16 * k0);
        }
    } else {
        const uintptr_t wb = (uintptr_t)a.w;
        const uintptr_t we = wb + (uintptr_t)a.n_out * (uintptr_t)a.row_bytes;
        const uintptr_t hi16 = (we & ~(uintptr_t)15) - 16;   // last whole granule
        const uintptr_t start = wb + (uintptr_t)row0 * (uintptr_t)a.row_bytes;
        const uintptr_t base16 = start & ~(uintptr_t)15;
        o0 = (uint32_t)(start & 15);
        const int ngr = (int)((o0 + (uint32_t)(R * a.row_bytes) + 15) / 16) + 1;
        for (int k0 = 64 * wave; k0 < ngr; k0 += 64 * W) {
            uintptr_t g = base16 + 16 * (uintptr_t)(k0 + lane);
            g = g > hi16 ? hi16 : g;
            dma16((const void *)g, rgb + 16 * k0);
        }
    }
    // The table (this thread's entries) and its exactness vote, while the
    // rows are in flight.
    {
        const bool exact = F::build_table(tab, threadIdx.x, 256 * NS);
        const bool any = __builtin_amdgcn_ballot_w64(!exact) != 0;
        if (lane == 0)
            *(volatile __attribute__((address_space(3))) uint32_t *)(size_t)(
                lds0 + F::kTable + cb_rg_region<F>(nb) + W * R * 4 + 4 * wave) = any ? 1u : 0u;
    }
    wait_vmcnt<0>();
    lds_barrier();   // the rows, the table and the votes

    float acc = 0.0f;
    const int row = row0 + r;
    if (b < nb) {
        const uint8_t *rg = smem + F::kTable;
        const uint32_t o = o0 + (uint32_t)((r * nb + b) * F::kBytes);
        switch (G) {
            case 0: acc = cb_rows_dot<F, 0>(a, rg, o, row, b, r, lane, xv); break;
            case 1: acc = cb_rows_dot<F, 1>(a, rg, o, row, b, r, lane, xv); break;
            case 2: acc = cb_rows_dot<F, 2>(a, rg, o, row, b, r, lane, xv); break;
            default: acc = cb_rows_dot<F, 3>(a, rg, o, row, b, r, lane, xv); break;
        }
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    float *red = (float *)(smem + F::kTable + cb_rg_region<F>(nb));
    if (lane < R) red[wave * R + lane] = acc;
    lds_barrier();
    if (wave != 0 || lane >= R) return;
    float total = red[lane];
#pragma unroll
    for (int w = 1; w < W; ++w) total += red[w * R + lane];
    const volatile __attribute__((address_space(3))) uint32_t *vote =
        (const volatile __attribute__((address_space(3))) uint32_t *)(size_t)(
            lds0 + F::kTable + cb_rg_region<F>(nb) + W * R * 4);
    uint32_t bad = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) bad |= vote[w];
    if (bad != 0u) total = __builtin_nanf("");
    if (row0 + lane < a.n_out) a.y[row0 + lane] = total;
}

template <class F>
hipError_t cb_rows_launch(const GemvArgs &a, const float *tab, hipStream_t s) {
    const dim3 g((a.n_out + kCbRgRows - 1) / kCbRgRows);
    if (a.nb <= 8)
        hipLaunchKernelGGL((cb_rows_kernel<F, 1>), g, dim3(256), cb_rg_lds<F>(a.nb, 4), s, a, tab);
    else if (a.nb <= 16)
        hipLaunchKernelGGL((cb_rows_kernel<F, 2>), g, dim3(512), cb_rg_lds<F>(a.nb, 8), s, a, tab);
    else
        hipLaunchKernelGGL((cb_rows_kernel<F, 3>), g, dim3(768), cb_rg_lds<F>(a.nb, 12), s, a, tab);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_iq3s_dequant(const uint8_t *src, const float *grid, float *dst, int64_t nblocks,
                               hipStream_t s) {
    int64_t groups = (nblocks + 3) / 4;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(iq3s_dequant_kernel, dim3((unsigned)groups), dim3(256), 0, s, src, grid, dst,
                       nblocks);
    return hipGetLastError();
}

hipError_t launch_iq4xs_dequant(const uint8_t *src, const float *table, float *dst,
                                int64_t nblocks, hipStream_t s) {
    int64_t groups = (nblocks + 3) / 4;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(iq4xs_dequant_kernel, dim3((unsigned)groups), dim3(256), 0, s, src, table,
                       dst, nblocks);
    return hipGetLastError();
}

hipError_t launch_cb_pack_tiles(int fmt, const uint8_t *src, uint8_t *dst, int nb, int n_out,
                                hipStream_t s) {
    const int64_t tiles = ((int64_t)n_out + kTileRows - 1) / kTileRows;
    const dim3 grid((unsigned)(tiles * nb)), block(256);
    if (fmt == kFmtIq3s)
        hipLaunchKernelGGL(cb_pack_tiles_kernel<Iq3sFmt>, grid, block, 0, s, src, dst, nb, n_out);
    else if (fmt == kFmtIq4xs)
        hipLaunchKernelGGL(cb_pack_tiles_kernel<Iq4xsFmt>, grid, block, 0, s, src, dst, nb, n_out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

int cb_stream_shape(int fmt, bool split) {
    if (fmt == kFmtIq3s) return cb_shape_f<Iq3sFmt>(split);
    if (fmt == kFmtIq4xs) return cb_shape_f<Iq4xsFmt>(split);
    return 0;
}

int cb_stream_slots(int fmt, bool tiled, int shape) {
    if (fmt == kFmtIq3s)
        return tiled ? cb_slots_any<Iq3sFmt, true>(shape) : cb_slots_any<Iq3sFmt, false>(shape);
    if (fmt == kFmtIq4xs)
        return tiled ? cb_slots_any<Iq4xsFmt, true>(shape) : cb_slots_any<Iq4xsFmt, false>(shape);
    return 0;
}

hipError_t launch_cb_stream(int fmt, bool tiled, int shape, const GroupArgs &g,
                            const GemvArgs &single, const float *tab, int nitems, hipStream_t s) {
    if (fmt == kFmtIq3s)
        return tiled ? cb_launch<Iq3sFmt, true>(shape, g, single, tab, nitems, s)
                     : cb_launch<Iq3sFmt, false>(shape, g, single, tab, nitems, s);
    if (fmt == kFmtIq4xs)
        return tiled ? cb_launch<Iq4xsFmt, true>(shape, g, single, tab, nitems, s)
                     : cb_launch<Iq4xsFmt, false>(shape, g, single, tab, nitems, s);
    return hipErrorInvalidValue;
}

bool cb_rows_fits(int nb) { return nb <= kCbRgMaxBlocks; }

hipError_t launch_cb_rows(int fmt, const GemvArgs &a, const float *tab, hipStream_t s) {
    if (a.nb > kCbRgMaxBlocks) return hipErrorInvalidValue;
    if (fmt == kFmtIq3s) return cb_rows_launch<Iq3sFmt>(a, tab, s);
    if (fmt == kFmtIq4xs) return cb_rows_launch<Iq4xsFmt>(a, tab, s);
    return hipErrorInvalidValue;
}

}  // namespace qwg
