// Q4_K kernels for gfx950: dequantization and the fused dequantize-GEMV/GEMM.
//
// Format: "用 Python 重写 picoLM" page, dequantize_q4_K listing. A 144-byte
// super-block holds fp16 d (bytes 0-1), fp16 dmin (2-3), twelve bytes of packed
// 6-bit scales/mins (4-15) and 128 quant bytes (16-143). Quant chunk c (bytes
// 16+32c .. +31) gives weights 64c+t from its low nibbles (sub-block 2c) and
// 64c+32+t from its high nibbles (sub-block 2c+1). Weight = d*sc_j*q - dmin*mn_j.
//
// GEMV design (one 64-row tile per workgroup, 4 wavefronts):
//   * lane r of every wavefront owns output row (tile*64 + r); wavefront g owns
//     quant chunk g (sub-blocks 2g, 2g+1) of every super-block, so all lanes of a
//     wavefront need the same 64 activations at any moment: they come through
//     scalar loads (SGPR operands), never through LDS or VGPRs;
//   * the tile's 64 x 144-byte blocks of one super-block column are fetched with
//     coalesced 16-byte loads (each row's block is contiguous) into registers one
//     column ahead, then written to a double-buffered LDS stage and read back per
//     lane (row stride 144 B = 36 dwords: conflict-free for 16-byte reads);
//   * a nibble is placed in an fp16 register half as a subnormal bit pattern
//     (value q*2^-24, or q*2^-20 for a high nibble masked in place), which
//     v_fma_mix_f32 widens exactly inside the FMA: one VALU op per weight;
//   * per sub-block the sum is factored: d*sc*sum(q*x) - dmin*mn*sum(x), with
//     sum(x) per 32-weight sub-block computed once per workgroup into LDS;
//   * a row's super-block range may be split over several workgroups (the
//     partial sums meet in tile_epilogue) so that small matrices still occupy
//     every compute unit.
#include "qwg_device.h"

namespace qwg {

namespace {

constexpr int kThreads = 256;                        // 4 wavefronts
constexpr int kStageBytes = kTileRows * kQ4kBytes;   // 9216: one super-block column of a tile
constexpr int kStageChunks = kStageBytes / 16;       // 576 16-byte chunks
static_assert(kStageChunks == 2 * kThreads + 64, "stage = two chunks per thread + one per lane of wavefront 0");

// Super-blocks whose per-sub-block activation sums fit the 16 KB sum buffer.
__host__ __device__ constexpr int sx_chunk_blocks(int nb_batch) { return 512 / nb_batch; }

// ------------------------------------------------------------------ dequant

// One wavefront per block: lane l produces weights 4l..4l+3 (all in sub-block
// l/8, quant chunk l/16, quant bytes 32*(l/16) + 4*(l%8) .. +3) and stores them
// as one 16-byte write, so a wavefront writes the block's 1 KB contiguously.
__global__ __launch_bounds__(256) void q4k_dequant_kernel(const uint8_t *__restrict__ src,
                                                          float *__restrict__ dst,
                                                          int64_t nblocks) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int j = lane >> 3;      // sub-block
    const int c = lane >> 4;      // quant chunk
    const int t4 = lane & 7;
    for (int64_t ib = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); ib < nblocks;
         ib += nwaves) {
        const uint8_t *b = src + ib * kQ4kBytes;
        const uint4 h = *(const uint4 *)b;
        const uint32_t qd = *(const uint32_t *)(b + 16 + 32 * c + 4 * t4);
        const float d = h2f_lo(h.x);
        const float dmin = h2f_hi(h.x);
        uint32_t sc, mn;
        if (j < 4) {
            sc = (h.y >> (8 * j)) & 63u;
            mn = (h.z >> (8 * j)) & 63u;
        } else {
            const int jj = j - 4;
            sc = ((h.w >> (8 * jj)) & 15u) | (((h.y >> (8 * jj + 6)) & 3u) << 4);
            mn = ((h.w >> (8 * jj + 4)) & 15u) | (((h.z >> (8 * jj + 6)) & 3u) << 4);
        }
        const uint32_t qb = (j & 1) ? (qd >> 4) : qd;
        // (d*sc)*q - dmin*mn in fp32, each operation rounded on its own.
        const float dsc = __fmul_rn(d, (float)sc);
        const float dmn = __fmul_rn(dmin, (float)mn);
        float4 o;
        o.x = __fsub_rn(__fmul_rn(dsc, (float)(qb & 15u)), dmn);
        o.y = __fsub_rn(__fmul_rn(dsc, (float)((qb >> 8) & 15u)), dmn);
        o.z = __fsub_rn(__fmul_rn(dsc, (float)((qb >> 16) & 15u)), dmn);
        o.w = __fsub_rn(__fmul_rn(dsc, (float)((qb >> 24) & 15u)), dmn);
        *(float4 *)(dst + ib * kQK + 4 * lane) = o;
    }
}

// ------------------------------------------------------------------ GEMV / GEMM

// Scale and min of sub-blocks 2G and 2G+1 from the packed bytes p[0..11]
// (h.y = p[0..3], h.z = p[4..7], h.w = p[8..11]). For j < 4 the six bits sit in
// byte j (scale) / byte j+4 (min); for j >= 4 the low nibble comes from byte
// j+4 and the top two bits from bits 6-7 of byte j-4 (scale) / byte j (min).
template <int G>
__device__ __forceinline__ void q4k_scales(const uint4 &h, uint32_t &sc0, uint32_t &sc1,
                                           uint32_t &mn0, uint32_t &mn1) {
    if constexpr (G < 2) {
        constexpr int s0 = 16 * G, s1 = 16 * G + 8;
        sc0 = (h.y >> s0) & 63u;
        sc1 = (h.y >> s1) & 63u;
        mn0 = (h.z >> s0) & 63u;
        mn1 = (h.z >> s1) & 63u;
    } else {
        constexpr int s0 = 16 * (G - 2), s1 = s0 + 8;
        sc0 = ((h.w >> s0) & 15u) | (((h.y >> (s0 + 6)) & 3u) << 4);
        sc1 = ((h.w >> s1) & 15u) | (((h.y >> (s1 + 6)) & 3u) << 4);
        mn0 = ((h.w >> (s0 + 4)) & 15u) | (((h.z >> (s0 + 6)) & 3u) << 4);
        mn1 = ((h.w >> (s1 + 4)) & 15u) | (((h.z >> (s1 + 6)) & 3u) << 4);
    }
}

// Wavefront G's share of one super-block for this lane's row: quant chunk G.
// xg points at x[256*b + 64*G] of batch element 0 (uniform across the wave).
template <int G, int NB>
__device__ __forceinline__ void q4k_chunk(const uint8_t *rowp, cfloat_p xg,
                                          int n_in, const float *sx, int sx_stride,
                                          uint32_t mlo, uint32_t mhi, float (&acc)[NB]) {
    const uint4 h = *(const uint4 *)rowp;
    const uint4 qa = *(const uint4 *)(rowp + 16 + 32 * G);
    const uint4 qb = *(const uint4 *)(rowp + 32 + 32 * G);
    uint32_t sc0, sc1, mn0, mn1;
    q4k_scales<G>(h, sc0, sc1, mn0, mn1);
    const float d = h2f_lo(h.x);
    const float dmin = h2f_hi(h.x);
    // Low nibbles enter as q*2^-24 and high nibbles as q*2^-20; fold 2^24 / 2^20
    // into the (exact) products d*sc.
    const float dsc0 = d * (float)(sc0 << 24);
    const float dsc1 = d * (float)(sc1 << 20);
    const float dmn0 = dmin * (float)mn0;
    const float dmn1 = dmin * (float)mn1;
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
        cfloat_p xb = xg + (int64_t)bt * n_in;
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t e = q[m] & mlo;            // bytes 0, 2: low nibbles
            const uint32_t o = (q[m] >> 8) & mlo;     // bytes 1, 3: low nibbles
            const uint32_t eh = q[m] & mhi;           // bytes 0, 2: high nibbles << 4
            const uint32_t oh = (q[m] >> 8) & mhi;    // bytes 1, 3: high nibbles << 4
            s0 = __builtin_fmaf(h2f_lo(e), xb[4 * m + 0], s0);
            s0 = __builtin_fmaf(h2f_lo(o), xb[4 * m + 1], s0);
            s0 = __builtin_fmaf(h2f_hi(e), xb[4 * m + 2], s0);
            s0 = __builtin_fmaf(h2f_hi(o), xb[4 * m + 3], s0);
            s1 = __builtin_fmaf(h2f_lo(eh), xb[32 + 4 * m + 0], s1);
            s1 = __builtin_fmaf(h2f_lo(oh), xb[32 + 4 * m + 1], s1);
            s1 = __builtin_fmaf(h2f_hi(eh), xb[32 + 4 * m + 2], s1);
            s1 = __builtin_fmaf(h2f_hi(oh), xb[32 + 4 * m + 3], s1);
        }
        const float sx0 = sx[bt * sx_stride + 2 * G];
        const float sx1 = sx[bt * sx_stride + 2 * G + 1];
        float a = acc[bt];
        a = __builtin_fmaf(dsc0, s0, a);
        a = __builtin_fmaf(dsc1, s1, a);
        a = __builtin_fmaf(-dmn0, sx0, a);
        a = __builtin_fmaf(-dmn1, sx1, a);
        acc[bt] = a;
    }
}

template <int G, int NB>
__device__ __forceinline__ void q4k_tile(const GemvArgs &a, uint8_t *smem, int tile, int split) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kb0 = (int)((int64_t)split * a.nb / a.splits);
    const int kb1 = (int)((int64_t)(split + 1) * a.nb / a.splits);
    const int nblk = kb1 - kb0;
    const int row0 = tile * kTileRows;

    uint8_t *stage = smem;                                     // [2][kStageBytes]
    float *sx = (float *)(smem + 2 * kStageBytes);             // [NB][8*chunk]
    // sum(x) is kept for at most kSxChunk(NB) super-blocks at a time.
    const int chunk = min(nblk, sx_chunk_blocks(NB));
    const int sx_stride = 8 * chunk;

    // 16-byte chunks this thread moves per stage: chunk c is byte 16*(c%9) of
    // the block of tile row c/9 (rows past n_out re-read the last row). Chunks
    // tid and tid+256 for everyone, tid+512 for wavefront 0 (576 in all).
    auto chunk_off = [&](int c) -> int64_t {
        const int r = c / 9;
        const int part = c - 9 * r;
        const int rg = min(row0 + r, a.n_out - 1);
        return (int64_t)rg * a.row_bytes + 16 * part;
    };
    const int64_t goff0 = chunk_off(tid);
    const int64_t goff1 = chunk_off(tid + kThreads);
    const int64_t goff2 = chunk_off(G == 0 ? tid + 2 * kThreads : tid);

    // sum(x) over each 32-weight sub-block of super-blocks [c0, c0 + chunk),
    // k ascending. The barrier that publishes it is the first one of the stage
    // loop below.
    auto sum_x = [&](int c0, int c1) {
        const int n = 8 * (c1 - c0);
        for (int j = tid; j < NB * n; j += kThreads) {
            const int bt = j / n;
            const int sb = j - bt * n;
            const float4 *xp = (const float4 *)(a.x + (int64_t)bt * a.n_in + 32 * (8 * c0 + sb));
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 v = xp[i];
                s += v.x;
                s += v.y;
                s += v.z;
                s += v.w;
            }
            sx[bt * sx_stride + sb] = s;
        }
    };

    uint4 r0, r1, r2 = make_uint4(0, 0, 0, 0);
    {
        const uint8_t *base = a.w + (int64_t)kb0 * kQ4kBytes;
        r0 = *(const uint4 *)(base + goff0);
        r1 = *(const uint4 *)(base + goff1);
        if constexpr (G == 0) r2 = *(const uint4 *)(base + goff2);
    }

    const uint32_t mlo = opaque(0x000F000Fu);
    const uint32_t mhi = opaque(0x00F000F0u);
    float acc[NB];
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) acc[bt] = 0.0f;

    int cend = kb0;
    for (int b = kb0; b < kb1; ++b) {
        if (b == cend) {
            // New sum(x) chunk; past the first, wait until every wavefront has
            // finished with the previous chunk's sums.
            if (b != kb0) __syncthreads();
            cend = min(b + chunk, kb1);
            sum_x(b, cend);
        }
        uint8_t *buf = stage + ((b - kb0) & 1) * kStageBytes;
        *(uint4 *)(buf + 16 * tid) = r0;
        *(uint4 *)(buf + 16 * (tid + kThreads)) = r1;
        if constexpr (G == 0) *(uint4 *)(buf + 16 * (tid + 2 * kThreads)) = r2;
        if (b + 1 < kb1) {
            const uint8_t *base = a.w + (int64_t)(b + 1) * kQ4kBytes;
            r0 = *(const uint4 *)(base + goff0);
            r1 = *(const uint4 *)(base + goff1);
            if constexpr (G == 0) r2 = *(const uint4 *)(base + goff2);
        }
        __syncthreads();
        cfloat_p xg = as_scalar(a.x) + (int64_t)kQK * b + 64 * G;
        q4k_chunk<G, NB>(buf + lane * kQ4kBytes, xg, a.n_in, sx + 8 * ((b - kb0) % chunk),
                         sx_stride, mlo, mhi, acc);
    }

    // Cross-wavefront sum of the four chunks, in chunk order. The red buffer
    // overlays stage 0, which nobody reads after the barrier below.
    __syncthreads();
    float *red = (float *)smem;  // [4][NB][64]
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) red[(G * NB + bt) * 64 + lane] = acc[bt];
    __syncthreads();
    if constexpr (G == 0) {
        float total[NB];
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) {
            float t = red[(0 * NB + bt) * 64 + lane];
            t += red[(1 * NB + bt) * 64 + lane];
            t += red[(2 * NB + bt) * 64 + lane];
            t += red[(3 * NB + bt) * 64 + lane];
            total[bt] = t;
        }
        tile_epilogue<NB>(a, tile, split, total);
    }
}

template <int NB>
__global__ __launch_bounds__(kThreads) void q4k_gemv_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tile = blockIdx.x / a.splits;
    const int split = blockIdx.x - tile * a.splits;
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
        case 0: q4k_tile<0, NB>(a, smem, tile, split); break;
        case 1: q4k_tile<1, NB>(a, smem, tile, split); break;
        case 2: q4k_tile<2, NB>(a, smem, tile, split); break;
        default: q4k_tile<3, NB>(a, smem, tile, split); break;
    }
}

}  // namespace

hipError_t launch_q4k_dequant(const uint8_t *src, float *dst, int64_t nblocks, hipStream_t s) {
    int64_t groups = (nblocks + 3) / 4;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(q4k_dequant_kernel, dim3((unsigned)groups), dim3(256), 0, s, src, dst,
                       nblocks);
    return hipGetLastError();
}

hipError_t launch_q4k_gemv(const GemvArgs &a, int batch, hipStream_t s) {
    if (batch < 1 || batch > 8) return hipErrorInvalidValue;
    int max_blk = (a.nb + a.splits - 1) / a.splits;
    if (max_blk > sx_chunk_blocks(batch)) max_blk = sx_chunk_blocks(batch);
    size_t lds = 2 * (size_t)kStageBytes + sizeof(float) * (size_t)batch * 8 * max_blk;
    const size_t red = sizeof(float) * 4 * (size_t)batch * 64;
    if (lds < red) lds = red;
    const dim3 grid((unsigned)(a.tiles * a.splits));
    switch (batch) {
        case 1: hipLaunchKernelGGL(q4k_gemv_kernel<1>, grid, dim3(kThreads), lds, s, a); break;
        case 2: hipLaunchKernelGGL(q4k_gemv_kernel<2>, grid, dim3(kThreads), lds, s, a); break;
        case 3: hipLaunchKernelGGL(q4k_gemv_kernel<3>, grid, dim3(kThreads), lds, s, a); break;
        case 4: hipLaunchKernelGGL(q4k_gemv_kernel<4>, grid, dim3(kThreads), lds, s, a); break;
        case 5: hipLaunchKernelGGL(q4k_gemv_kernel<5>, grid, dim3(kThreads), lds, s, a); break;
        case 6: hipLaunchKernelGGL(q4k_gemv_kernel<6>, grid, dim3(kThreads), lds, s, a); break;
        case 7: hipLaunchKernelGGL(q4k_gemv_kernel<7>, grid, dim3(kThreads), lds, s, a); break;
        case 8: hipLaunchKernelGGL(q4k_gemv_kernel<8>, grid, dim3(kThreads), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qwg
