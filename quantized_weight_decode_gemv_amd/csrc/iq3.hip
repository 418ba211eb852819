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
// GEMV design (one 64-row tile per workgroup, 4 wavefronts):
//   * lane r owns row tile*64 + r; wavefront g owns sub-blocks 2g and 2g+1 of
//     every block, so activations are wave-uniform and come through scalar loads;
//   * the tile's 64 blocks of one column are staged through LDS as 25-dword
//     windows starting at the dword below each block (blocks are only 2-byte
//     aligned); lanes re-align their words with v_alignbyte;
//   * the grid is expanded once per workgroup into a sign-folded fp16 table
//     T[s][idx] = (+-g0, +-g1, +-g2, +-g3) for the 16 sign patterns s of a group
//     of four weights, so four weights cost one v_perm (table index from the
//     index byte and the sign nibble), one shift, one 8-byte LDS read and four
//     v_fma_mix_f32;
//   * the eighth sign of each 8-weight group is rebuilt for all four groups of a
//     word at once with byte-parallel XOR folding.
#include "qwg_device.h"

namespace qwg {

namespace {

constexpr int kThreads = 256;
constexpr int kWinDwords = 25;                              // 100-byte window per block
constexpr int kStageDwords = kTileRows * kWinDwords;        // 1600
constexpr int kStageBytes = kStageDwords * 4;               // 6400
constexpr int kTableBytes = 16 * 256 * 8;                   // 32 KB sign-folded grid
constexpr int kLoadsPerThread = (kStageDwords + kThreads - 1) / kThreads;  // 7

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

// ------------------------------------------------------------------ dequant

// One wavefront per block: lane l produces weights 4l..4l+3, i.e. the four
// magnitudes of grid row idx[l] of sub-block l/8.
__global__ __launch_bounds__(256) void iq3_dequant_kernel(const uint8_t *__restrict__ src,
                                                          const float *__restrict__ grid,
                                                          float *__restrict__ dst,
                                                          int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int ib = lane >> 3;         // sub-block
    const int t0 = 4 * (lane & 7);    // first weight of this lane within the sub-block
    for (int64_t blk = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
         blk < nblocks; blk += nwaves) {
        const uint8_t *b = src + blk * kIq3Bytes;
        const float d = h2f_lo(load_u16(b + 96));
        const uint32_t word = load_u32_a2(b + 64 + 4 * ib);
        const uint32_t code = word >> 28;
        const float db = __fmul_rn(__fmul_rn(d, 0.5f + (float)code), 0.5f);
        const uint32_t s8 = iq3_signs(word);
        const float4 g = *(const float4 *)(grid + 4 * b[lane]);
        float4 o;
        o.x = __fmul_rn(((s8 >> (t0 + 0)) & 1u) ? -g.x : g.x, db);
        o.y = __fmul_rn(((s8 >> (t0 + 1)) & 1u) ? -g.y : g.y, db);
        o.z = __fmul_rn(((s8 >> (t0 + 2)) & 1u) ? -g.z : g.z, db);
        o.w = __fmul_rn(((s8 >> (t0 + 3)) & 1u) ? -g.w : g.w, db);
        *(float4 *)(dst + blk * kQK + 4 * lane) = o;
    }
}

// ------------------------------------------------------------------ GEMV

// Wavefront G's two sub-blocks (2G, 2G+1) of one block for this lane's row.
// win: this row's 25-dword window (LDS), sh: byte offset of the block in it
// (0 or 2). xg: x[256*b + 64*G] (wave-uniform). table: sign-folded fp16 grid.
template <int G>
__device__ __forceinline__ float iq3_chunk(const uint32_t *win, uint32_t sh,
                                           cfloat_p xg, const uint8_t *table,
                                           float acc) {
    // Block dwords 4G..4G+3 (indices) and 16+2G, 17+2G (words), re-aligned.
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = win[4 * G + i];
    uint32_t v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = win[16 + 2 * G + i];
    const uint32_t dwin = win[24];
    uint32_t idx[4], words[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) idx[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
#pragma unroll
    for (int i = 0; i < 2; ++i) words[i] = __builtin_amdgcn_alignbyte(v[i + 1], v[i], sh);
    const float d = h2f_lo(dwin >> (8 * sh));
    const float dq = d * 0.25f;   // d*(0.5+code)*0.5 == (d/4)*(2*code+1), exact
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t word = words[half];
        const uint32_t s8 = iq3_signs(word);
        const uint32_t ne = s8 & 0x0F0F0F0Fu;          // sign nibbles of groups 0,2,4,6
        const uint32_t no = (s8 >> 4) & 0x0F0F0F0Fu;   // groups 1,3,5,7
        const float db = dq * (float)(2u * (word >> 28) + 1u);
        cfloat_p xs = xg + 32 * half;
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // table index = nibble*256 + idx: byte 0 = index byte k, byte 1 = nibble k
            const uint32_t sel = (uint32_t)(k & 3) | ((uint32_t)(4 + (k >> 1)) << 8) | 0x0C0C0000u;
            const uint32_t ti = __builtin_amdgcn_perm((k & 1) ? no : ne, idx[2 * half + (k >> 2)], sel);
            const uint2 e = *(const uint2 *)(table + (ti << 3));
            s = __builtin_fmaf(h2f_lo(e.x), xs[4 * k + 0], s);
            s = __builtin_fmaf(h2f_hi(e.x), xs[4 * k + 1], s);
            s = __builtin_fmaf(h2f_lo(e.y), xs[4 * k + 2], s);
            s = __builtin_fmaf(h2f_hi(e.y), xs[4 * k + 3], s);
        }
        acc = __builtin_fmaf(db, s, acc);
    }
    return acc;
}

template <int G>
__device__ __forceinline__ void iq3_tile(const GemvArgs &a, uint8_t *smem, int tile, int split) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kb0 = (int)((int64_t)split * a.nb / a.splits);
    const int kb1 = (int)((int64_t)(split + 1) * a.nb / a.splits);
    const int row0 = tile * kTileRows;

    uint8_t *table = smem;                                   // [16][256] x 8 bytes
    uint32_t *stage = (uint32_t *)(smem + kTableBytes);      // [2][64][25] dwords

    // Sign-folded fp16 table: entry (s, i) = grid row i with component c negated
    // when bit c of s is set.
    for (int e = tid; e < 16 * 256; e += kThreads) {
        const int s = e >> 8, i = e & 255;
        const float4 g = *(const float4 *)(a.grid + 4 * i);
        const float gv[4] = {g.x, g.y, g.z, g.w};
        uint32_t hb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const _Float16 hv = (_Float16)(((s >> c) & 1) ? -gv[c] : gv[c]);
            hb[c] = __builtin_bit_cast(uint16_t, hv);
        }
        *(uint2 *)(table + 8 * e) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    }

    // Staging: dword c of the stage is dword c%25 of the window of tile row c/25.
    // The window of the block at byte offset o starts at o & ~3; when o is a
    // multiple of 4 its last dword would cover two bytes past the block, so that
    // dword is read as 16 bits (the two bytes of d) to stay inside the buffer.
    int64_t rowoff[kLoadsPerThread];
    int dwi[kLoadsPerThread];
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
        const int c = tid + kThreads * i;
        const int r = c / kWinDwords;
        dwi[i] = c - kWinDwords * r;
        rowoff[i] = (int64_t)min(row0 + r, a.n_out - 1) * a.row_bytes;
    }
    // Windows are aligned on absolute addresses, so every window dword is a
    // naturally aligned 32-bit load (the weights are at least 2-byte aligned).
    const uintptr_t wbase = (uintptr_t)a.w;
    auto load_stage = [&](int b, uint32_t (&dst)[kLoadsPerThread]) {
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i) {
            if (tid + kThreads * i < kStageDwords) {
                const uintptr_t o = wbase + (uintptr_t)(rowoff[i] + (int64_t)b * kIq3Bytes);
                const uintptr_t p = (o & ~(uintptr_t)3) + 4 * dwi[i];
                if (dwi[i] == kWinDwords - 1 && (o & 3) == 0)
                    dst[i] = load_u16((const uint8_t *)p);
                else
                    dst[i] = *(const uint32_t *)p;
            }
        }
    };

    uint32_t r[kLoadsPerThread];
    load_stage(kb0, r);
    float acc = 0.0f;
    const int64_t my_rowoff = (int64_t)min(row0 + lane, a.n_out - 1) * a.row_bytes;
    for (int b = kb0; b < kb1; ++b) {
        uint32_t *buf = stage + ((b - kb0) & 1) * kStageDwords;
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i)
            if (tid + kThreads * i < kStageDwords) buf[tid + kThreads * i] = r[i];
        if (b + 1 < kb1) load_stage(b + 1, r);
        __syncthreads();
        const uint32_t sh = (uint32_t)((wbase + (uintptr_t)(my_rowoff + (int64_t)b * kIq3Bytes)) & 3);
        acc = iq3_chunk<G>(buf + lane * kWinDwords, sh, as_scalar(a.x) + (int64_t)kQK * b + 64 * G,
                           table, acc);
    }

    __syncthreads();
    float *red = (float *)stage;  // [4][64], overlays stage 0
    red[G * 64 + lane] = acc;
    __syncthreads();
    if constexpr (G == 0) {
        float total[1];
        float t = red[lane];
        t += red[64 + lane];
        t += red[128 + lane];
        t += red[192 + lane];
        total[0] = t;
        tile_epilogue<1>(a, tile, split, total);
    }
}

__global__ __launch_bounds__(kThreads) void iq3_gemv_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tile = blockIdx.x / a.splits;
    const int split = blockIdx.x - tile * a.splits;
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
        case 0: iq3_tile<0>(a, smem, tile, split); break;
        case 1: iq3_tile<1>(a, smem, tile, split); break;
        case 2: iq3_tile<2>(a, smem, tile, split); break;
        default: iq3_tile<3>(a, smem, tile, split); break;
    }
}

}  // namespace

hipError_t launch_iq3_dequant(const uint8_t *src, const float *grid, float *dst,
                              int64_t nblocks, hipStream_t s) {
    int64_t groups = (nblocks + 3) / 4;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(iq3_dequant_kernel, dim3((unsigned)groups), dim3(256), 0, s, src, grid,
                       dst, nblocks);
    return hipGetLastError();
}

hipError_t launch_iq3_gemv(const GemvArgs &a, hipStream_t s) {
    const size_t lds = kTableBytes + 2 * (size_t)kStageBytes;
    hipLaunchKernelGGL(iq3_gemv_kernel, dim3((unsigned)(a.tiles * a.splits)), dim3(kThreads), lds,
                       s, a);
    return hipGetLastError();
}

}  // namespace qwg
