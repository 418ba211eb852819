// Q4_K kernels for gfx950: dequantization and the fused dequantize-GEMV/GEMM.
//
// Format: "用 Python 重写 picoLM" page, dequantize_q4_K listing. A 144-byte
// super-block holds fp16 d (bytes 0-1), fp16 dmin (2-3), twelve bytes of packed
// 6-bit scales/mins (4-15) and 128 quant bytes (16-143). Quant chunk c (bytes
// 16+32c .. +31) gives weights 64c+t from its low nibbles (sub-block 2c) and
// 64c+32+t from its high nibbles (sub-block 2c+1). Weight = d*sc_j*q - dmin*mn_j.
//
// GEMV design (one 64-row tile per workgroup of W = 4, 8 or 16 wavefronts):
//   * lane r of every wavefront owns output row tile*64 + r; wavefront 4j+G owns
//     quant chunk G (sub-blocks 2G, 2G+1) of the j-th super-block of each
//     pipeline stage, so all lanes of a wavefront need the same 64 activations:
//     they come through scalar loads as SGPR operands, never through LDS/VGPRs;
//   * each stage (64 rows x W/4 super-blocks) is copied into LDS by LDS-DMA
//     (global_load_lds_dwordx4, 16 bytes per lane, coalesced: a row's block is
//     contiguous) while the previous stage is computed; every wavefront counts
//     its own copies (s_waitcnt vmcnt) before the stage barrier;
//   * a nibble is placed in an fp16 register half as a subnormal bit pattern
//     (value q*2^-24, or q*2^-20 for a high nibble masked in place), which
//     v_fma_mix_f32 widens exactly inside the FMA: one VALU op per weight;
//   * per sub-block the sum is factored: d*sc*sum(q*x) - dmin*mn*sum(x), with
//     sum(x) per 32-weight sub-block computed once per workgroup into LDS;
//   * the W wavefronts' row sums meet in LDS; for small matrices a row's
//     super-block range may also be split over several workgroups (the partial
//     sums meet in tile_epilogue) so that every compute unit gets work. A
//     grouped launch runs many independent GEMVs in one grid.
#include "qwg_device.h"
#include "q4k_dot.h"

namespace qwg {

namespace {

constexpr int kStageBytes = kTileRows * kQ4kBytes;   // 9216: one super-block column of a tile

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
        // written once, never re-read here: the non-temporal hint (measured on the 32000 x 2048
        // matrix: 66.0 -> 41.0 us, 4.5 -> 7.3 TB/s of bytes read and written)
        __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, (f32x4 *)(dst + ib * kQK + 4 * lane));
    }
}

// ------------------------------------------------------------------ tile layout

// One workgroup per (tile, block column): the 64 rows' block b (row-major
// source) written back to back; rows past n_out become zero blocks.
__global__ __launch_bounds__(256) void q4k_pack_tiles_kernel(const uint8_t *__restrict__ src,
                                                             uint8_t *__restrict__ dst, int nb,
                                                             int n_out) {
    const int b = blockIdx.x % nb;
    const int tile = blockIdx.x / nb;
    const int64_t row_bytes = (int64_t)nb * kQ4kBytes;
    uint8_t *out = dst + (int64_t)blockIdx.x * kStageBytes;
    for (int k = threadIdx.x; k < kStageBytes / 16; k += blockDim.x) {
        const int r = tile * kTileRows + k / 9;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < n_out) v = *(const uint4 *)(src + r * row_bytes + b * kQ4kBytes + 16 * (k % 9));
        *(uint4 *)(out + 16 * k) = v;
    }
}

// ------------------------------------------------------------------ GEMV / GEMM

// One pipeline stage holds BPS = W/4 super-block columns of the 64-row tile,
// laid out [block j][row r][144 B]: a row stride of 144 B (36 dwords) puts the
// 16-byte reads of 16 consecutive lanes in distinct banks. Wavefront w = 4j+G
// copies rows 16G..16G+15 of block j into the stage (144 chunks of 16 bytes:
// LDS-DMA instructions of 64, 64 and 16 lanes) and computes quant chunk G of
// block j for all 64 rows. Two stage buffers: the copy of stage s+1 runs while
// stage s is computed.
template <int G, int NB, int W>
__device__ __forceinline__ void q4k_tile(const GemvArgs &a, uint8_t *smem, int tile, int split) {
    constexpr int BPS = W / 4;
    constexpr int SBYTES = BPS * kStageBytes;
    // sum(x) is kept for SXB super-blocks at a time (16 KB), a multiple of BPS.
    constexpr int SXB = ((512 / NB) / BPS) * BPS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = __builtin_amdgcn_readfirstlane(tid >> 8);   // block within the stage
    const int wave = 4 * j + G;
    const int kb0 = (int)((int64_t)split * a.nb / a.splits);
    const int kb1 = (int)((int64_t)(split + 1) * a.nb / a.splits);
    const int nblk = kb1 - kb0;
    const int nst = (nblk + BPS - 1) / BPS;
    const int row0 = tile * kTileRows;

    float *sx = (float *)(smem + 2 * SBYTES);               // [NB][8 * min(nblk, SXB)]
    const int sx_stride = 8 * min(nblk, SXB);

    // This wavefront's 16-byte chunks k = 64i + lane (i = 0, 1) and 128 + lane
    // (lanes 0..15): tile row 16G + k/9, byte 16*(k%9) of the block. Rows past
    // n_out re-read the last row.
    int64_t goff[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int k = (i < 2 || lane < 16) ? 64 * i + lane : 128;
        const int r = 16 * G + k / 9;
        goff[i] = (int64_t)min(row0 + r, a.n_out - 1) * a.row_bytes + 16 * (k % 9);
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem + j * kStageBytes + 2304 * G;
    auto issue = [&](int s) {
        const int b = kb0 + s * BPS + j;
        if (b < kb1) {
            const uint8_t *base = a.w + (int64_t)b * kQ4kBytes;
            const uint32_t dst = lds_base + (s & 1) * SBYTES;
            dma16(base + goff[0], dst);
            dma16(base + goff[1], dst + 1024);
            if (lane < 16) dma16(base + goff[2], dst + 2048);
        }
    };

    // sum(x) over each 32-weight sub-block of super-blocks [c0, c1), k ascending.
    auto sum_x = [&](int c0, int c1) {
        const int n = 8 * (c1 - c0);
        for (int q = tid; q < NB * n; q += W * 64) {
            const int bt = q / n;
            const int sb = q - bt * n;
            const float4 *xp = (const float4 *)(a.x + (int64_t)bt * a.n_in + 32 * (8 * c0 + sb));
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 v = xp[i];
                sum += v.x;
                sum += v.y;
                sum += v.z;
                sum += v.w;
            }
            sx[bt * sx_stride + sb] = sum;
        }
    };

    const uint32_t mlo = opaque(0x000F000Fu);
    const uint32_t mhi = opaque(0x00F000F0u);
    float acc[NB];
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) acc[bt] = 0.0f;

    issue(0);
    for (int s = 0; s < nst; ++s) {
        // New sum(x) chunk: every wavefront is past the previous stage's barrier.
        if ((s * BPS) % SXB == 0) sum_x(kb0 + s * BPS, min(kb0 + s * BPS + SXB, kb1));
        if (s + 1 < nst) issue(s + 1);
        // This wavefront's copies of stage s are done once at most the copies of
        // stage s+1 (3 instructions, if it issued any) are outstanding.
        if (s + 1 < nst && kb0 + (s + 1) * BPS + j < kb1)
            wait_vmcnt<3>();
        else
            wait_vmcnt<0>();
        lds_barrier();  // stage s and the sums are complete for every wavefront
        const int b = kb0 + s * BPS + j;
        if (b < kb1) {
            const uint8_t *rowp = smem + (s & 1) * SBYTES + j * kStageBytes + lane * kQ4kBytes;
            const float *sxb = sx + 8 * ((b - kb0) % SXB) + 2 * G;
            float sx0[NB], sx1[NB];
#pragma unroll
            for (int bt = 0; bt < NB; ++bt) {
                sx0[bt] = sxb[bt * sx_stride];
                sx1[bt] = sxb[bt * sx_stride + 1];
            }
            q4k_chunk<G, NB>(rowp, as_scalar(a.x) + (int64_t)kQK * b + 64 * G, a.n_in, sx0, sx1,
                             mlo, mhi, acc);
        }
        lds_barrier();  // stage buffer s&1 and the sums may be overwritten
    }

    // Cross-wavefront sum in wavefront order (blocks j, then chunks G). The
    // buffer overlays stage 0, idle after the last barrier.
    float *red = (float *)smem;  // [W][NB][64]
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) red[(wave * NB + bt) * 64 + lane] = acc[bt];
    lds_barrier();
    if (wave == 0) {
        float total[NB];
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) {
            float t = red[bt * 64 + lane];
            for (int w = 1; w < W; ++w) t += red[(w * NB + bt) * 64 + lane];
            total[bt] = t;
        }
        tile_epilogue<NB>(a, tile, split, total);
    }
}

template <int NB, int W>
__device__ __forceinline__ void q4k_dispatch(const GemvArgs &a, uint8_t *smem, int tile, int split) {
    switch (__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3)) {
        case 0: q4k_tile<0, NB, W>(a, smem, tile, split); break;
        case 1: q4k_tile<1, NB, W>(a, smem, tile, split); break;
        case 2: q4k_tile<2, NB, W>(a, smem, tile, split); break;
        default: q4k_tile<3, NB, W>(a, smem, tile, split); break;
    }
}

template <int NB, int W>
__global__ __launch_bounds__(W * 64) void q4k_gemv_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tile = blockIdx.x / a.splits;
    q4k_dispatch<NB, W>(a, smem, tile, blockIdx.x - tile * a.splits);
}

// ------------------------------------------------------------------ batched GEMM on matrix cores
//
// For 2 <= batch <= 8 the product is a dense contraction: per 32-weight
// sub-block, P[b][r] = sum_k x[b][k] q[r][k] for every batch row b and weight
// row r, then y[b][r] += d*sc * P - dmin*mn * sum_k x[b][k]. The sums go to
// v_mfma_f32_16x16x32_bf16 exactly:
//  * weights enter as bf16(16 + q) = 0x4180 | q << 3 (a mask and an OR per
//    pair), so the MFMA forms sum (16 + q) x and the 16*sum(x) is taken off in
//    the scale step: y += d*sc * C - (16*d*sc + dmin*mn) * S;
//  * x enters as three bf16 parts x = hi + mid + lo, each the top 16 bits of
//    the remainder (exact for normal fp32), accumulated into the same fp32 C;
//  * S = sum x over the sub-block comes from the same MFMA with all-ones weights.
// Every product (4-bit integer times 8-bit significand) is exact; only the fp32
// accumulation rounds, as in the scalar path.
//
// Operand layout of the 16x16x32 instruction (measured): lane l holds A[l%16][k]
// and B[k][l%16] for k = 8*(l/16) .. 8*(l/16)+7, and C[4*(l/16)+i][l%16].
// Here A = x: row m of A is batch m%8 of sub-block 2G (m < 8) or 2G+1 (m >= 8);
// B = the weights of 16 tile rows (column n = row). Wavefront G of a 4-wavefront
// workgroup computes quant chunk G (sub-blocks 2G, 2G+1) of every super-block
// for all 64 rows of the tile (4 groups of 16): C1 = A B(2G), C2 = A B(2G+1);
// lanes 0-31 keep C1's rows 0-7, lanes 32-63 C2's rows 8-15, so each lane ends
// with one weight row, one sub-block and four batch rows.
//
// A stage holds H super-block columns (H = 1: 4 wavefronts; H = 2: 8, the
// second four taking the odd columns of the workgroup's range): per column the
// 64 rows' blocks (9216 B, copied as in the tiled engine), then per wavefront
// its 64 activations of each of the 8 batch rows (2 KB, 16-byte granule of
// (batch b, k/4 = c) at slot 16*(c%8) + 8*(c/8) + b, so that the 16 lanes of a
// k-group read 16 distinct bank quads). Batch rows past `batch` copy row 0 and
// are zeroed in A. R stages form a ring, R - 1 of them in flight while one is
// computed. A workgroup does only a few stages and each is a chain of
// dependent LDS, MFMA and ALU steps, so the time goes to latency; H = 2 halves
// the stages and doubles the wavefronts that hide it.
constexpr int kXSlice = 2048;
constexpr int kMfmaStage = kStageBytes + 4 * kXSlice;   // 17408
constexpr int kMfmaScales = 1024;                        // per wavefront: [64 rows][2][d*sc, offset]

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// bf16 from the top halves of two fp32 bit patterns: (lo >> 16) | (hi & 0xFFFF0000).
__device__ __forceinline__ uint32_t bf16_pack(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Three-part split of 8 activations into A fragments (slot order 0,2,1,3,4,6,5,7,
// matching q4k_bf16_quants).
__device__ __forceinline__ void split_x(const float (&v)[8], bool live, u32x4_t &a_hi,
                                        u32x4_t &a_mid, u32x4_t &a_lo) {
    uint32_t h[8], m[8], l[8];
    const uint32_t top = opaque(0xFFFF0000u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = live ? v[i] : 0.0f;
        h[i] = __builtin_bit_cast(uint32_t, x) & top;
        const float r = x - __builtin_bit_cast(float, h[i]);
        m[i] = __builtin_bit_cast(uint32_t, r) & top;
        l[i] = __builtin_bit_cast(uint32_t, r - __builtin_bit_cast(float, m[i])) & top;
    }
    constexpr int ord[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_hi[i] = bf16_pack(h[ord[2 * i]], h[ord[2 * i + 1]]);
        a_mid[i] = bf16_pack(m[ord[2 * i]], m[ord[2 * i + 1]]);
        a_lo[i] = bf16_pack(l[ord[2 * i]], l[ord[2 * i + 1]]);
    }
}

// B fragments of 8 quant bytes e0..e7 (one k-group of a row): low nibbles
// (sub-block 2G) and high nibbles (2G+1) as bf16(16 + q), in slot order
// (e0,e2), (e1,e3), (e4,e6), (e5,e7).
__device__ __forceinline__ void q4k_bf16_quants(uint2 e, uint32_t mask, uint32_t bias,
                                                u32x4_t &b_lo, u32x4_t &b_hi) {
    const uint32_t d[2] = {e.x, e.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        b_lo[2 * i] = ((d[i] << 3) & mask) | bias;
        b_lo[2 * i + 1] = ((d[i] >> 5) & mask) | bias;
        b_hi[2 * i] = ((d[i] >> 1) & mask) | bias;
        b_hi[2 * i + 1] = ((d[i] >> 9) & mask) | bias;
    }
}

// Wait until this wavefront's copies of a stage have landed while the copies of
// `newer` later stages (five instructions each) may still be in flight.
__device__ __forceinline__ void wait_stage_copies(int newer) {
    switch (__builtin_amdgcn_readfirstlane(newer)) {
        case 1: wait_vmcnt<5>(); break;
        case 2: wait_vmcnt<10>(); break;
        case 3: wait_vmcnt<15>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

template <int G, int NB, int R, int H, bool TL>
__device__ __forceinline__ void q4k_mfma_tile(const GemvArgs &a, uint8_t *smem, int tile, int split,
                                              int h) {
    static_assert(R >= 2 && R <= 4, "ring of two to four stages");
    static_assert(H == 1 || H == 2, "one or two columns per stage");
    constexpr int kStage = H * kMfmaStage;
    const int lane = threadIdx.x & 63;
    const int kb0 = (int)((int64_t)split * a.nb / a.splits);
    const int kb1 = (int)((int64_t)(split + 1) * a.nb / a.splits);
    const int nst = (kb1 - kb0 + H - 1) / H;
    const int row0 = tile * kTileRows;

    // Copy lanes: rows 16G..16G+15 of the column, 16-byte chunk k of them at
    // LDS byte 2304G + 16k. Row-major weights: rows past n_out re-read the
    // last row. Tile layout (TL): the column is one contiguous 9216-byte run
    // (rows past n_out are zero blocks there).
    int64_t goff[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int k = (i < 2 || lane < 16) ? 64 * i + lane : 128;
        const int r = 16 * G + k / 9;
        goff[i] = TL ? (int64_t)(2304 * G + 16 * k)
                     : (int64_t)min(row0 + r, a.n_out - 1) * a.row_bytes + 16 * (k % 9);
    }
    const uint8_t *wtile = a.w + (TL ? (int64_t)tile * a.nb * kStageBytes : 0);
    int64_t xoff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int sl = 64 * t + lane;
        const int bt = sl & 7;
        const int c = 8 * ((sl >> 3) & 1) + (sl >> 4);
        xoff[t] = (int64_t)(bt < NB ? bt : 0) * a.n_in + 64 * G + 4 * c;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const int wave = 4 * h + G;
    const uint32_t wdst = lds0 + kStageBytes * h + 2304 * G;
    const uint32_t xdst = lds0 + H * kStageBytes + kXSlice * wave;
    // Column of this wavefront in step s. With two columns per stage, the last
    // step of an odd range has none for h = 1: that
    // wavefront copies the range's last column again (five copies per stage
    // keep the wait counts uniform) and skips the math.
    auto column = [&](int s) { return kb0 + H * s + h; };
    // Activation slots of batch rows past NB are zeroed in A: not copied.
    const bool xcopy = NB == 8 || (lane & 7) < NB;
    auto issue = [&](int s) {
        const int b = min(column(s), kb1 - 1);
        const uint32_t off = (uint32_t)(s % R) * kStage;
        if constexpr (TL) {
            // whole lines read once: the non-temporal hint, as in the stream engine
            const uint8_t *wb = wtile + (int64_t)b * kStageBytes;
            dma16_stream(wb + goff[0], wdst + off);
            dma16_stream(wb + goff[1], wdst + off + 1024);
            if (lane < 16) dma16_stream(wb + goff[2], wdst + off + 2048);
        } else {
            // plain copies: the next stage reads the neighbouring 144-byte block
            // of each row, often from the same line; the non-temporal hint
            // measured 0.4-0.8 us slower on the LM head
            const uint8_t *wb = a.w + (int64_t)b * kQ4kBytes;
            dma16(wb + goff[0], wdst + off);
            dma16(wb + goff[1], wdst + off + 1024);
            if (lane < 16) dma16(wb + goff[2], wdst + off + 2048);
        }
        const float *xb = a.x + (int64_t)kQK * b;
        if (xcopy) {
            dma16(xb + xoff[0], xdst + off);
            dma16(xb + xoff[1], xdst + off + 1024);
        }
    };

    // A-operand role of this lane and its activation slots
    const int am = lane & 15;          // A row: batch am%8, sub-block 2G + am/8
    const int kg = lane >> 4;          // k-group: k = 8kg .. 8kg+7
    const bool alive = (am & 7) < NB;
    const uint32_t xslot0 = 16u * (2 * kg) + 8u * (am >> 3) + (am & 7);
    // C role: weight row n of each 16-row group, sub-block parity, batch rows 4(kg&1)+i
    const int n = lane & 15;
    const bool upper = lane >= 32;

    float *scales = (float *)(smem + R * kStage + kMfmaScales * wave);
    const uint32_t mask = opaque(0x00780078u);
    const uint32_t bias = opaque(0x41804180u);
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = zero4;

    for (int s = 0; s < R - 1 && s < nst; ++s) issue(s);
    for (int s = 0; s < nst; ++s) {
        if (s + R - 1 < nst) issue(s + R - 1);   // into the slot computed in step s - 1
        wait_stage_copies(min(R - 1, nst - 1 - s));
        lds_barrier();
        if (H == 1 || column(s) < kb1) {
            const uint8_t *stage = smem + (s % R) * kStage + kStageBytes * h;
            // Scale terms of sub-blocks 2G and 2G+1 for every tile row, decoded once
            // (lane r: row r) and read back below by the lanes that hold that row.
            {
                const uint4 h = *(const uint4 *)(stage + lane * kQ4kBytes);
                uint32_t sc0, sc1, mn0, mn1;
                q4k_scales<G>(h, sc0, sc1, mn0, mn1);
                const float d = h2f_lo(h.x);
                const float dmin = h2f_hi(h.x);
                const float dsc0 = d * (float)sc0;
                const float dsc1 = d * (float)sc1;
                float4 t;
                t.x = dsc0;
                t.y = __builtin_fmaf(dmin, (float)mn0, 16.0f * dsc0);
                t.z = dsc1;
                t.w = __builtin_fmaf(dmin, (float)mn1, 16.0f * dsc1);
                *(float4 *)(scales + 4 * lane) = t;
                // (read back by other lanes of this wavefront: LDS keeps a wavefront's order)
                asm volatile("" ::: "memory");
            }
            const float *xs = (const float *)(smem + (s % R) * kStage + H * kStageBytes + kXSlice * wave);
            float xv[8];
            const float4 x0 = *(const float4 *)(xs + 4 * xslot0);
            const float4 x1 = *(const float4 *)(xs + 4 * (xslot0 + 16));
            xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
            xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
            u32x4_t ah, am_, al;
            split_x(xv, alive, ah, am_, al);
            f32x4_t sx = mfma_bf16(ah, ones, zero4);
            sx = mfma_bf16(am_, ones, sx);
            sx = mfma_bf16(al, ones, sx);
    #pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint8_t *rowp = stage + (16 * g + n) * kQ4kBytes;
                const uint2 e = *(const uint2 *)(rowp + 16 + 32 * G + 8 * kg);
                u32x4_t b_lo, b_hi;
                q4k_bf16_quants(e, mask, bias, b_lo, b_hi);
                f32x4_t c1 = mfma_bf16(ah, b_lo, zero4);
                c1 = mfma_bf16(am_, b_lo, c1);
                c1 = mfma_bf16(al, b_lo, c1);
                f32x4_t c2 = mfma_bf16(ah, b_hi, zero4);
                c2 = mfma_bf16(am_, b_hi, c2);
                c2 = mfma_bf16(al, b_hi, c2);
                const float2 so = *(const float2 *)(scales + 4 * (16 * g + n) + 2 * (int)upper);
                const float dsc = so.x;
                const float off = so.y;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float c = upper ? c2[i] : c1[i];
                    float v = __builtin_fmaf(dsc, c, acc[g][i]);
                    acc[g][i] = __builtin_fmaf(-off, sx[i], v);
                }
            }
        }
        lds_barrier();  // slot s % R may be overwritten
    }

    // Sub-blocks 2G and 2G+1 (lanes l and l^32), then the wavefronts in order
    // through LDS (overlaying stage 0, idle after the last barrier).
    float *red = (float *)smem;  // [wave][batch 8][row 64]
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = acc[g][i] + __shfl_xor(acc[g][i], 32);
            const int bt = 4 * (kg & 1) + i;
            if (!upper && bt < NB) red[(wave * 8 + bt) * 64 + 16 * g + n] = v;
        }
    }
    lds_barrier();
    if (wave == 0) {
        float total[NB];
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) {
            float t = red[bt * 64 + lane];
#pragma unroll
            for (int w = 1; w < 4 * H; ++w) t += red[(w * 8 + bt) * 64 + lane];
            total[bt] = t;
        }
        tile_epilogue<NB>(a, tile, split, total);
    }
}

template <int NB, int R, int H, bool TL>
__global__ __launch_bounds__(256 * H) void q4k_mfma_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tile = blockIdx.x / a.splits;
    const int split = blockIdx.x - tile * a.splits;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = H == 2 ? w >> 2 : 0;
    switch (w & 3) {
        case 0: q4k_mfma_tile<0, NB, R, H, TL>(a, smem, tile, split, h); break;
        case 1: q4k_mfma_tile<1, NB, R, H, TL>(a, smem, tile, split, h); break;
        case 2: q4k_mfma_tile<2, NB, R, H, TL>(a, smem, tile, split, h); break;
        default: q4k_mfma_tile<3, NB, R, H, TL>(a, smem, tile, split, h); break;
    }
}

// Batched grouped launch on the matrix cores: one workgroup per position of the
// group's work list (a 64-row tile of a member, or a hole; no splits; members
// of `batch` activation rows), the problem and tile found through the list
// with scalar loads, then the tile pipeline above with a 2-stage ring.
template <int NB, int H, bool TL>
__global__ __launch_bounds__(256 * H) void q4k_mfma_group_kernel(GroupArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t pi = ((cu32_p)g.map)[blockIdx.x];
    if (pi == kNoItem) return;   // a hole of the work list
    GemvArgs a;
    load_args(a, (cargs_p)g.problems + pi);
    const int tile = g.tile != nullptr ? (int)((cu32_p)g.tile)[blockIdx.x] : blockIdx.x - a.wg_begin;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = H == 2 ? w >> 2 : 0;
    switch (w & 3) {
        case 0: q4k_mfma_tile<0, NB, 2, H, TL>(a, smem, tile, 0, h); break;
        case 1: q4k_mfma_tile<1, NB, 2, H, TL>(a, smem, tile, 0, h); break;
        case 2: q4k_mfma_tile<2, NB, 2, H, TL>(a, smem, tile, 0, h); break;
        default: q4k_mfma_tile<3, NB, 2, H, TL>(a, smem, tile, 0, h); break;
    }
}

// Grouped launch (one workgroup per item): each workgroup reads its problem
// index and descriptor with scalar loads, then runs the same tile pipeline.

template <int W>
__global__ __launch_bounds__(W * 64) void q4k_group_kernel(GroupArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    GemvArgs a;
    load_args(a, (cargs_p)g.problems + ((cu32_p)g.map)[blockIdx.x]);
    const int local = blockIdx.x - a.wg_begin;
    const int tile = local / a.splits;
    q4k_dispatch<1, W>(a, smem, tile, local - tile * a.splits);
}

// ------------------------------------------------------------------ stream engine
//
// Persistent variant for batch 1: a grid of about one workgroup per LDS slot of
// the chip walks a list of "items" (one 64-row tile of one matrix, all or part
// of its super-block range), item k, k + gridDim.x, ... . The LDS ring of R
// stages runs ahead across item boundaries, so a workgroup's copy engine never
// idles between tiles. Each stage copy also brings the 64 activations of every
// wavefront's quant chunk (lanes 16..31 of its third DMA instruction), from
// which the wavefront forms its two 32-weight activation sums with a DPP
// reduction: no per-item prologue and no shared sum buffer.
template <int W, int R>
struct StreamCfg {
    static constexpr int kBps = W / 4;
    static constexpr int kQuarter = 16 * kQ4kBytes + 256;   // 16 rows + 64 activations
    static constexpr int kBlock = 4 * kQuarter;             // 10240
    static constexpr int kSlot = kBps * kBlock;
    static constexpr int kRed = R * kSlot;                  // [W][64] fp32 row sums
    static constexpr int kLds = kRed + W * 64 * 4;
};

// One item as seen by a cursor: one 64-row tile over super-blocks [kb0, kb1).
// Without SPLIT an item is the whole row (kb0 = 0, kb1 = nb). With SPLIT, item
// index `local` of a problem with `splits` ranges is tile local / splits, range
// local % splits, and the partial sums meet in tile_epilogue (prob: the
// problem's descriptor index, -1 for a single GEMV).
struct Item {
    const uint8_t *w;
    const float *x;
    float *y;
    int64_t row_bytes;
    int n_out;
    int nb;
    int nst;   // stages = ceil((kb1 - kb0) / BPS)
    int row0;
    int layout;
    int kb0, kb1, split, prob;
};

template <int BPS, bool SPLIT>
__device__ __forceinline__ void load_item(Item &it, int k, const GroupArgs &g, const GemvArgs &single) {
    if constexpr (!SPLIT) {
        if (g.problems == nullptr) {
            it.w = single.w;
            it.x = single.x;
            it.y = single.y;
            it.row_bytes = single.row_bytes;
            it.n_out = single.n_out;
            it.nb = single.nb;
            it.row0 = k * kTileRows;
            it.layout = single.layout;
        } else {
            const cargs_p pa = (cargs_p)g.problems + ((cu32_p)g.map)[k];
            it.w = pa->w;
            it.x = pa->x;
            it.y = pa->y;
            it.row_bytes = pa->row_bytes;
            it.n_out = pa->n_out;
            it.nb = pa->nb;
            it.row0 = (g.tile != nullptr ? (int)((cu32_p)g.tile)[k] : k - pa->wg_begin) * kTileRows;
            it.layout = pa->layout;
        }
        it.kb0 = 0;
        it.kb1 = it.nb;
        it.split = 0;
        it.prob = -1;
        it.nst = (it.nb + BPS - 1) / BPS;
    } else {
        int local, splits;
        if (g.problems == nullptr) {
            it.w = single.w;
            it.x = single.x;
            it.y = single.y;
            it.row_bytes = single.row_bytes;
            it.n_out = single.n_out;
            it.nb = single.nb;
            it.layout = single.layout;
            local = k;
            it.prob = -1;
            splits = single.splits;
        } else {
            const int pi = (int)((cu32_p)g.map)[k];
            const cargs_p pa = (cargs_p)g.problems + pi;
            it.w = pa->w;
            it.x = pa->x;
            it.y = pa->y;
            it.row_bytes = pa->row_bytes;
            it.n_out = pa->n_out;
            it.nb = pa->nb;
            it.layout = pa->layout;
            local = g.tile != nullptr ? (int)((cu32_p)g.tile)[k] : k - pa->wg_begin;
            it.prob = pi;
            splits = pa->splits;
        }
        const int tile = local / splits;
        it.split = local - tile * splits;
        it.row0 = tile * kTileRows;
        it.kb0 = it.split * it.nb / splits;
        it.kb1 = (it.split + 1) * it.nb / splits;
        it.nst = (it.kb1 - it.kb0 + BPS - 1) / BPS;
    }
}

template <int G, int W, int R, bool SPLIT>
__device__ __forceinline__ void q4k_stream(const GroupArgs &g, const GemvArgs &single, int nitems,
                                           uint8_t *smem) {
    static_assert(R >= 2 && R <= 3, "ring of two or three stages");
    using C = StreamCfg<W, R>;
    constexpr int BPS = C::kBps;
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const int wave = 4 * j + G;
    const int stride = gridDim.x;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // This wavefront's copy lanes: chunks k = 64i + lane of its 16 rows (row
    // 16G + k/9, byte 16*(k%9)); lanes 16..31 of the third instruction copy the
    // 64 activations of quant chunk G instead (4 per lane).
    int crow[3], cpart[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int k = (i < 2 || lane < 16) ? 64 * i + lane : 128;
        crow[i] = 16 * G + k / 9;
        cpart[i] = 16 * (k % 9);
    }
    const int64_t xoff = 4 * (64 * G + 4 * (lane - 16));   // bytes, lanes 16..31

    int kc = skip_holes(blockIdx.x, stride, nitems, g);  // item being computed
    if (kc >= nitems) return;
    Item c;
    load_item<BPS, SPLIT>(c, kc, g, single);

    // copy cursor: next stage sd of item kd goes to ring slot slot_d
    int kd = kc, sd = 0, slot_d = 0, pending = 0;
    Item d = c;
    // Block b of this wavefront's copy granule i comes from dbase + b*dstride +
    // doff[i]: in the row layout the rows are row_bytes apart (rows past n_out
    // repeat the last row); in the tile layout a tile's block column is 9216
    // contiguous bytes in copy order.
    int64_t doff[3];
    const uint8_t *dbase = nullptr;
    int dstride = 0;
    auto prep_copy = [&]() {
        if (d.layout == kLayoutTiles) {
            dbase = d.w + (int64_t)(d.row0 / kTileRows) * d.nb * kStageBytes;
            dstride = kStageBytes;
#pragma unroll
            for (int i = 0; i < 3; ++i) doff[i] = (int64_t)crow[i] * kQ4kBytes + cpart[i];
        } else {
            dbase = d.w;
            dstride = kQ4kBytes;
#pragma unroll
            for (int i = 0; i < 3; ++i)
                doff[i] = (int64_t)min(d.row0 + crow[i], d.n_out - 1) * d.row_bytes + cpart[i];
        }
    };
    prep_copy();
    uint32_t flags = 0;  // bit k: this wavefront's copies are in ring slot k
    auto issue_next = [&]() {
        if (kd >= nitems) return;
        const int b = d.kb0 + sd * BPS + j;
        if (b < d.kb1) {
            const uint32_t base = lds0 + slot_d * C::kSlot + j * C::kBlock + G * C::kQuarter;
            const uint8_t *wb = dbase + (int64_t)b * dstride;
            // Tile-layout stages are whole lines read once: stream them past the
            // caches. Row-major stages share straddled lines with the next stage,
            // which the hint would evict (measured 110 -> 133 us on the C5 stream).
            if (d.layout == kLayoutTiles) {
                dma16_stream(wb + doff[0], base);
                dma16_stream(wb + doff[1], base + 1024);
            } else {
                dma16(wb + doff[0], base);
                dma16(wb + doff[1], base + 1024);
            }
            if (lane < 32) {
                const uint8_t *src = lane < 16 ? wb + doff[2]
                                               : (const uint8_t *)d.x + (int64_t)(kQK * 4) * b + xoff;
                dma16(src, base + 2048);
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
                load_item<BPS, SPLIT>(d, kd, g, single);
                prep_copy();
            }
        }
    };
#pragma unroll
    for (int i = 0; i < R - 1; ++i) issue_next();

    const uint32_t mlo = opaque(0x000F000Fu);
    const uint32_t mhi = opaque(0x00F000F0u);
    float *red = (float *)(smem + C::kRed);
    int slot_c = 0;
    for (;;) {
        float acc[1] = {0.0f};
        for (int s = 0; s < c.nst; ++s) {
            const int b = c.kb0 + s * BPS + j;
            // With three slots, the next stage may already be in flight: allow
            // its three copies (if this wavefront issued any) to stay pending.
            const int nxt = slot_c + 1 == R ? 0 : slot_c + 1;
            if (R == 3 && pending > 1 && ((flags >> nxt) & 1u))
                wait_vmcnt<3>();
            else
                wait_vmcnt<0>();
            lds_barrier();   // stage in slot_c complete for every wavefront
            issue_next();    // refill the slot computed in the previous step
            if (b < c.kb1) {
                const uint8_t *blk = smem + slot_c * C::kSlot + j * C::kBlock;
                const uint8_t *rowp = blk + (lane >> 4) * C::kQuarter + (lane & 15) * kQ4kBytes;
                const float xs = ((const float *)(blk + G * C::kQuarter + 16 * kQ4kBytes))[lane];
                const float hs = half_wave_sum(xs);
                const float sx0[1] = {__builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hs), 16))};
                const float sx1[1] = {__builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hs), 48))};
                q4k_chunk<G, 1>(rowp, as_scalar(c.x) + (int64_t)kQK * b + 64 * G, 0, sx0, sx1, mlo,
                                mhi, acc);
            }
            --pending;
            slot_c = nxt;
        }
        // row sums of the W wavefronts, in wavefront order
        red[wave * 64 + lane] = acc[0];
        lds_barrier();
        if (wave == 0) {
            float tsum = red[lane];
            for (int w = 1; w < W; ++w) tsum += red[w * 64 + lane];
            if (SPLIT) {
                GemvArgs ea;
                if (c.prob >= 0)
                    load_args(ea, (cargs_p)g.problems + c.prob);
                else
                    ea = single;
                const float total[1] = {tsum};
                tile_epilogue<1>(ea, c.row0 / kTileRows, c.split, total);
            } else if (c.row0 + lane < c.n_out) {
                c.y[c.row0 + lane] = tsum;
            }
        }
        kc = skip_holes(kc + stride, stride, nitems, g);
        if (kc >= nitems) break;
        load_item<BPS, SPLIT>(c, kc, g, single);
    }
}

// The SGPR budget keeps seven 4-wavefront workgroups resident per CU: the x
// operands of a quant chunk take 64 SGPRs, and measured on gfx950 a kernel
// whose last SGPR is s94 or higher fits only six wavefronts per SIMD (the
// occupancy query still reports seven, so a grid sized by it would leave a
// seventh of the workgroups waiting for a slot). A budget of 96 ends at s87;
// the few spills go to VGPR lanes outside the inner loop.
//
// SPLIT: items may cover part of a row (problems with splits > 1), whose sums
// meet through the problem's partial-sum workspace; the variant without it is
// the one that streams whole rows (no epilogue round trip, fewer registers).
template <int W, int R, bool SPLIT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_num_sgpr(96))) void q4k_stream_kernel(
    GroupArgs g, GemvArgs single, int nitems) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    switch (__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3)) {
        case 0: q4k_stream<0, W, R, SPLIT>(g, single, nitems, smem); break;
        case 1: q4k_stream<1, W, R, SPLIT>(g, single, nitems, smem); break;
        case 2: q4k_stream<2, W, R, SPLIT>(g, single, nitems, smem); break;
        default: q4k_stream<3, W, R, SPLIT>(g, single, nitems, smem); break;
    }
}

// ------------------------------------------------------------------ batched stream on matrix cores
//
// Persistent form of the matrix-core pipeline above for 2 <= batch <= 8: a grid
// of resident 4-wavefront workgroups walks the item list as the batch-1 stream
// engine does (item k, k + gridDim.x, ...), and an R-slot ring of stages runs
// ahead across item boundaries, so the copies of the next tile's columns are in
// flight while a tile ends. A stage is one super-block column of the tile (the
// 64 rows' blocks, 9216 B) and each wavefront's 64 activations of every batch
// row (2 KB, laid out as above); the arithmetic per stage is the one above. A
// tile's row sums meet in LDS over the stage slot just computed (not refilled
// before the next barrier) and leave through tile_epilogue (SPLIT) or straight
// stores.
template <int R>
struct MStreamCfg {
    static constexpr int kSlot = kMfmaStage;                  // weights, then [wave] x slices
    static constexpr int kLds = R * kSlot;
};

template <int G, int NB, int R, bool SPLIT>
__device__ __forceinline__ void q4k_mstream(const GroupArgs &g, const GemvArgs &single, int nitems,
                                            uint8_t *smem) {
    static_assert(R >= 2 && R <= 4, "ring of two to four stages");
    using C = MStreamCfg<R>;
    const int lane = threadIdx.x & 63;
    const int stride = gridDim.x;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // Weight copy lanes as in the pipeline above: chunk k = 64i + lane (i < 2,
    // or lanes 0..15 for i = 2) of rows 16G..16G+15, LDS byte 2304G + 16k.
    int crow[3], cpart[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int k = (i < 2 || lane < 16) ? 64 * i + lane : 128;
        crow[i] = 16 * G + k / 9;
        cpart[i] = 16 * (k % 9);
    }
    // Activation copy lanes: 16-byte granule t of this lane holds x[bt][256b +
    // 64G + 4c .. +3] (batch rows past NB copy row 0 and are zeroed in A).
    int xbt[2], xc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int sl = 64 * t + lane;
        const int bt = sl & 7;
        xbt[t] = bt < NB ? bt : 0;
        xc[t] = 8 * ((sl >> 3) & 1) + (sl >> 4);
    }

    int kc = skip_holes(blockIdx.x, stride, nitems, g);
    if (kc >= nitems) return;
    Item c;
    load_item<1, SPLIT>(c, kc, g, single);

    int kd = kc, sd = 0, slot_d = 0, pending = 0;
    Item d = c;
    int64_t doff[3], xoff[2];
    const uint8_t *dbase = nullptr;
    int dstride = 0;
    auto prep_copy = [&]() {
        if (d.layout == kLayoutTiles) {
            dbase = d.w + (int64_t)(d.row0 / kTileRows) * d.nb * kStageBytes;
            dstride = kStageBytes;
#pragma unroll
            for (int i = 0; i < 3; ++i) doff[i] = (int64_t)crow[i] * kQ4kBytes + cpart[i];
        } else {
            dbase = d.w;
            dstride = kQ4kBytes;
#pragma unroll
            for (int i = 0; i < 3; ++i)
                doff[i] = (int64_t)min(d.row0 + crow[i], d.n_out - 1) * d.row_bytes + cpart[i];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
            xoff[t] = 4 * ((int64_t)xbt[t] * d.nb * kQK + 64 * G + 4 * xc[t]);
    };
    prep_copy();
    // Every stage is five copy instructions per wavefront (three of weights,
    // two of activations), so waits count stages.
    auto issue_next = [&]() {
        if (kd >= nitems) return;
        const int b = d.kb0 + sd;
        const uint32_t base = lds0 + slot_d * C::kSlot;
        const uint8_t *wb = dbase + (int64_t)b * dstride;
        const uint32_t wdst = base + 2304 * G;
        if (d.layout == kLayoutTiles) {
            dma16_stream(wb + doff[0], wdst);
            dma16_stream(wb + doff[1], wdst + 1024);
            if (lane < 16) dma16_stream(wb + doff[2], wdst + 2048);
        } else {
            dma16(wb + doff[0], wdst);
            dma16(wb + doff[1], wdst + 1024);
            if (lane < 16) dma16(wb + doff[2], wdst + 2048);
        }
        const uint8_t *xb = (const uint8_t *)d.x + (int64_t)(kQK * 4) * b;
        const uint32_t xdst = base + kStageBytes + kXSlice * G;
        dma16(xb + xoff[0], xdst);
        dma16(xb + xoff[1], xdst + 1024);
        ++pending;
        slot_d = slot_d + 1 == R ? 0 : slot_d + 1;
        if (++sd == d.nst) {
            sd = 0;
            kd = skip_holes(kd + stride, stride, nitems, g);
            if (kd < nitems) {
                load_item<1, SPLIT>(d, kd, g, single);
                prep_copy();
            }
        }
    };
#pragma unroll
    for (int i = 0; i < R - 1; ++i) issue_next();

    // A-operand role of this lane and its activation slots; C role (as above)
    const int am = lane & 15;
    const int kg = lane >> 4;
    const bool alive = (am & 7) < NB;
    const uint32_t xslot0 = 16u * (2 * kg) + 8u * (am >> 3) + (am & 7);
    const int n = lane & 15;
    const bool upper = lane >= 32;
    const uint32_t mask = opaque(0x00780078u);
    const uint32_t bias = opaque(0x41804180u);
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const f32x4_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

    int slot_c = 0;
    for (;;) {
        f32x4_t acc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = zero4;
        int last = slot_c;
        for (int s = 0; s < c.nst; ++s) {
            // copies of the stages issued after this one may stay in flight
            wait_stage_copies(pending - 1);
            lds_barrier();   // stage in slot_c complete for every wavefront
            issue_next();    // refill the slot computed in the previous step
            const uint8_t *stage = smem + slot_c * C::kSlot;
            // Every LDS read of the step first, then one wait: the headers and
            // quant bytes of this lane's four rows (16q + n) and its
            // activation slots. Each lane decodes the scales of its own rows
            // and sub-block (no round trip through LDS to share them).
            uint4 hd[4];
            uint2 e[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint8_t *rowp = stage + (16 * q + n) * kQ4kBytes;
                hd[q] = *(const uint4 *)rowp;
                e[q] = *(const uint2 *)(rowp + 16 + 32 * G + 8 * kg);
            }
            const float *xs = (const float *)(stage + kStageBytes + kXSlice * G);
            const float4 x0 = *(const float4 *)(xs + 4 * xslot0);
            const float4 x1 = *(const float4 *)(xs + 4 * (xslot0 + 16));
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            u32x4_t ah, am_, al;
            split_x(xv, alive, ah, am_, al);
            f32x4_t sx = mfma_bf16(ah, ones, zero4);
            sx = mfma_bf16(am_, ones, sx);
            sx = mfma_bf16(al, ones, sx);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4_t b_lo, b_hi;
                q4k_bf16_quants(e[q], mask, bias, b_lo, b_hi);
                f32x4_t c1 = mfma_bf16(ah, b_lo, zero4);
                c1 = mfma_bf16(am_, b_lo, c1);
                c1 = mfma_bf16(al, b_lo, c1);
                f32x4_t c2 = mfma_bf16(ah, b_hi, zero4);
                c2 = mfma_bf16(am_, b_hi, c2);
                c2 = mfma_bf16(al, b_hi, c2);
                uint32_t sc0, sc1, mn0, mn1;
                q4k_scales<G>(hd[q], sc0, sc1, mn0, mn1);
                const float dsc = h2f_lo(hd[q].x) * (float)(upper ? sc1 : sc0);
                const float off =
                    __builtin_fmaf(h2f_hi(hd[q].x), (float)(upper ? mn1 : mn0), 16.0f * dsc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float cv = upper ? c2[i] : c1[i];
                    const float v = __builtin_fmaf(dsc, cv, acc[q][i]);
                    acc[q][i] = __builtin_fmaf(-off, sx[i], v);
                }
            }
            --pending;
            last = slot_c;
            slot_c = slot_c + 1 == R ? 0 : slot_c + 1;
        }
        // Sub-blocks 2G and 2G+1 (lanes l and l^32), then the wavefronts in
        // order, through the slot just computed: every wavefront is past its
        // reads, and it is refilled only after the next barrier.
        lds_barrier();
        float *red = (float *)(smem + last * C::kSlot);   // [wave][batch 8][row 64]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = acc[q][i] + __shfl_xor(acc[q][i], 32);
                const int bt = 4 * (kg & 1) + i;
                if (!upper && bt < NB) red[(G * 8 + bt) * 64 + 16 * q + n] = v;
            }
        }
        lds_barrier();
        if (G == 0) {
            float total[NB];
#pragma unroll
            for (int bt = 0; bt < NB; ++bt) {
                float t = red[bt * 64 + lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) t += red[(w * 8 + bt) * 64 + lane];
                total[bt] = t;
            }
            if (SPLIT) {
                GemvArgs ea;
                if (c.prob >= 0)
                    load_args(ea, (cargs_p)g.problems + c.prob);
                else
                    ea = single;
                tile_epilogue<NB>(ea, c.row0 / kTileRows, c.split, total);
            } else if (c.row0 + lane < c.n_out) {
#pragma unroll
                for (int bt = 0; bt < NB; ++bt) c.y[(int64_t)bt * c.n_out + c.row0 + lane] = total[bt];
            }
        }
        kc = skip_holes(kc + stride, stride, nitems, g);
        if (kc >= nitems) break;
        load_item<1, SPLIT>(c, kc, g, single);
    }
}

template <int NB, int R, bool SPLIT>
__global__ __launch_bounds__(256) void q4k_mstream_kernel(GroupArgs g, GemvArgs single, int nitems) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    switch (__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3)) {
        case 0: q4k_mstream<0, NB, R, SPLIT>(g, single, nitems, smem); break;
        case 1: q4k_mstream<1, NB, R, SPLIT>(g, single, nitems, smem); break;
        case 2: q4k_mstream<2, NB, R, SPLIT>(g, single, nitems, smem); break;
        default: q4k_mstream<3, NB, R, SPLIT>(g, single, nitems, smem); break;
    }
}

template <int W>
size_t q4k_lds_bytes(int batch, int max_blk) {
    const int sxb = ((512 / batch) / (W / 4)) * (W / 4);
    if (max_blk > sxb) max_blk = sxb;
    return 2 * (size_t)(W / 4) * kStageBytes + sizeof(float) * (size_t)batch * 8 * max_blk;
}

}  // namespace

hipError_t launch_q4k_dequant(const uint8_t *src, float *dst, int64_t nblocks, hipStream_t s) {
    int64_t groups = (nblocks + 3) / 4;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(q4k_dequant_kernel, dim3((unsigned)groups), dim3(256), 0, s, src, dst,
                       nblocks);
    return hipGetLastError();
}

hipError_t launch_q4k_pack_tiles(const uint8_t *src, uint8_t *dst, int nb, int n_out, hipStream_t s) {
    const int64_t tiles = ((int64_t)n_out + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL(q4k_pack_tiles_kernel, dim3((unsigned)(tiles * nb)), dim3(256), 0, s, src,
                       dst, nb, n_out);
    return hipGetLastError();
}

template <int W>
hipError_t launch_q4k_gemv_w(const GemvArgs &a, int batch, hipStream_t s) {
    const size_t lds = q4k_lds_bytes<W>(batch, (a.nb + a.splits - 1) / a.splits);
    const dim3 grid((unsigned)(a.tiles * a.splits)), block(W * 64);
    switch (batch) {
        case 1: hipLaunchKernelGGL((q4k_gemv_kernel<1, W>), grid, block, lds, s, a); break;
        case 2: hipLaunchKernelGGL((q4k_gemv_kernel<2, W>), grid, block, lds, s, a); break;
        case 3: hipLaunchKernelGGL((q4k_gemv_kernel<3, W>), grid, block, lds, s, a); break;
        case 4: hipLaunchKernelGGL((q4k_gemv_kernel<4, W>), grid, block, lds, s, a); break;
        case 5: hipLaunchKernelGGL((q4k_gemv_kernel<5, W>), grid, block, lds, s, a); break;
        case 6: hipLaunchKernelGGL((q4k_gemv_kernel<6, W>), grid, block, lds, s, a); break;
        case 7: hipLaunchKernelGGL((q4k_gemv_kernel<7, W>), grid, block, lds, s, a); break;
        case 8: hipLaunchKernelGGL((q4k_gemv_kernel<8, W>), grid, block, lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_q4k_gemv(const GemvArgs &a, int batch, int waves, hipStream_t s) {
    switch (waves) {
        case 4: return launch_q4k_gemv_w<4>(a, batch, s);
        case 8: return launch_q4k_gemv_w<8>(a, batch, s);
        case 16: return launch_q4k_gemv_w<16>(a, batch, s);
        default: return hipErrorInvalidValue;
    }
}

template <int W, int R>
int stream_residency(int *cus_out) {
    using C = StreamCfg<W, R>;
    struct Residency {
        int per_cu, cus;
    };
    // Queried once per process (a function-local static: initialised once even
    // when several host threads make the first call together).
    static const Residency r = [] {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, q4k_stream_kernel<W, R, false>,
                                                         W * 64, C::kLds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        return Residency{per_cu, cus};
    }();
    *cus_out = r.cus;
    return r.per_cu;
}

template <int W, int R>
hipError_t launch_stream_wr(const GroupArgs &g, const GemvArgs &single, int nitems, bool split,
                            hipStream_t s) {
    using C = StreamCfg<W, R>;
    int cus = 0;
    const int per_cu = stream_residency<W, R>(&cus);
    int grid = per_cu * cus;
    if (grid > nitems) grid = nitems;
    if (split)
        hipLaunchKernelGGL((q4k_stream_kernel<W, R, true>), dim3((unsigned)grid), dim3(W * 64),
                           C::kLds, s, g, single, nitems);
    else
        hipLaunchKernelGGL((q4k_stream_kernel<W, R, false>), dim3((unsigned)grid), dim3(W * 64),
                           C::kLds, s, g, single, nitems);
    return hipGetLastError();
}

hipError_t launch_q4k_stream(const GroupArgs &g, const GemvArgs &single, int nitems, int waves,
                             int ring, bool split, hipStream_t s) {
    switch (waves * 10 + ring) {
        case 42: return launch_stream_wr<4, 2>(g, single, nitems, split, s);
        case 43: return launch_stream_wr<4, 3>(g, single, nitems, split, s);
        case 82: return launch_stream_wr<8, 2>(g, single, nitems, split, s);
        case 83: return launch_stream_wr<8, 3>(g, single, nitems, split, s);
        case 162: return launch_stream_wr<16, 2>(g, single, nitems, split, s);
        case 163: return launch_stream_wr<16, 3>(g, single, nitems, split, s);
        default: return hipErrorInvalidValue;
    }
}

template <int R, int H, bool TL>
hipError_t launch_mfma_rh(const GemvArgs &a, int batch, hipStream_t s) {
    const size_t lds = (size_t)R * H * kMfmaStage + 4 * H * kMfmaScales;
    const dim3 grid((unsigned)(a.tiles * a.splits)), block(256 * H);
    switch (batch) {
#define QWG_MFMA_CASE(nb) \
    case nb: hipLaunchKernelGGL((q4k_mfma_kernel<nb, R, H, TL>), grid, block, lds, s, a); break;
        QWG_MFMA_CASE(2) QWG_MFMA_CASE(3) QWG_MFMA_CASE(4) QWG_MFMA_CASE(5) QWG_MFMA_CASE(6)
        QWG_MFMA_CASE(7) QWG_MFMA_CASE(8)
#undef QWG_MFMA_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_q4k_mfma(const GemvArgs &a, int batch, int ring, int cols, bool tiled,
                           hipStream_t s) {
    if (tiled) {   // tile layout: 2-stage ring only
        if (ring != 2) return hipErrorInvalidValue;
        return cols == 2 ? launch_mfma_rh<2, 2, true>(a, batch, s)
                         : launch_mfma_rh<2, 1, true>(a, batch, s);
    }
    switch (cols * 10 + ring) {
        case 12: return launch_mfma_rh<2, 1, false>(a, batch, s);
        case 13: return launch_mfma_rh<3, 1, false>(a, batch, s);
        case 14: return launch_mfma_rh<4, 1, false>(a, batch, s);
        case 22: return launch_mfma_rh<2, 2, false>(a, batch, s);
        default: return hipErrorInvalidValue;
    }
}

template <int H, bool TL>
hipError_t launch_mfma_group_h(const GroupArgs &g, int nwg, int batch, hipStream_t s) {
    const size_t lds = 2 * (size_t)H * kMfmaStage + 4 * H * kMfmaScales;
    const dim3 grid((unsigned)nwg), block(256 * H);
    switch (batch) {
#define QWG_MFMA_CASE(nb) \
    case nb: hipLaunchKernelGGL((q4k_mfma_group_kernel<nb, H, TL>), grid, block, lds, s, g); break;
        QWG_MFMA_CASE(2) QWG_MFMA_CASE(3) QWG_MFMA_CASE(4) QWG_MFMA_CASE(5) QWG_MFMA_CASE(6)
        QWG_MFMA_CASE(7) QWG_MFMA_CASE(8)
#undef QWG_MFMA_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_q4k_mfma_group(const GroupArgs &g, int nwg, int batch, int cols, bool tiled,
                                 hipStream_t s) {
    if (nwg < 1) return hipErrorInvalidValue;
    if (tiled)
        return cols == 2 ? launch_mfma_group_h<2, true>(g, nwg, batch, s)
                         : launch_mfma_group_h<1, true>(g, nwg, batch, s);
    return cols == 2 ? launch_mfma_group_h<2, false>(g, nwg, batch, s)
                     : launch_mfma_group_h<1, false>(g, nwg, batch, s);
}

// Resident workgroups of the batched matrix-core stream (ring R) on the current
// device, queried once per process.
template <int R>
int mstream_slots_r() {
    static const int slots = [] {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, q4k_mstream_kernel<8, R, true>,
                                                         256, MStreamCfg<R>::kLds) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        return per_cu * cus;
    }();
    return slots;
}

int q4k_mstream_slots(int ring) {
    switch (ring) {
        case 2: return mstream_slots_r<2>();
        case 3: return mstream_slots_r<3>();
        case 4: return mstream_slots_r<4>();
        default: return 0;
    }
}

template <int R, bool SPLIT>
hipError_t launch_mstream_rs(const GroupArgs &g, const GemvArgs &single, int nitems, int batch,
                             hipStream_t s) {
    int n = mstream_slots_r<R>();
    if (n > nitems) n = nitems;
    const dim3 grid((unsigned)n), block(256);
    const size_t lds = MStreamCfg<R>::kLds;
    switch (batch) {
#define QWG_MSTREAM_CASE(nb)                                                                     \
    case nb:                                                                                     \
        hipLaunchKernelGGL((q4k_mstream_kernel<nb, R, SPLIT>), grid, block, lds, s, g, single,   \
                           nitems);                                                              \
        break;
        QWG_MSTREAM_CASE(2) QWG_MSTREAM_CASE(3) QWG_MSTREAM_CASE(4) QWG_MSTREAM_CASE(5)
        QWG_MSTREAM_CASE(6) QWG_MSTREAM_CASE(7) QWG_MSTREAM_CASE(8)
#undef QWG_MSTREAM_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_q4k_mstream(const GroupArgs &g, const GemvArgs &single, int nitems, int batch,
                              int ring, bool split, hipStream_t s) {
    if (nitems < 1) return hipErrorInvalidValue;
    switch (ring * 2 + (split ? 1 : 0)) {
        case 4: return launch_mstream_rs<2, false>(g, single, nitems, batch, s);
        case 5: return launch_mstream_rs<2, true>(g, single, nitems, batch, s);
        case 6: return launch_mstream_rs<3, false>(g, single, nitems, batch, s);
        case 7: return launch_mstream_rs<3, true>(g, single, nitems, batch, s);
        case 8: return launch_mstream_rs<4, false>(g, single, nitems, batch, s);
        case 9: return launch_mstream_rs<4, true>(g, single, nitems, batch, s);
        default: return hipErrorInvalidValue;
    }
}

int q4k_stream_residency(int waves, int ring, int *cus) {
    switch (waves * 10 + ring) {
        case 42: return stream_residency<4, 2>(cus);
        case 43: return stream_residency<4, 3>(cus);
        case 82: return stream_residency<8, 2>(cus);
        case 83: return stream_residency<8, 3>(cus);
        case 162: return stream_residency<16, 2>(cus);
        case 163: return stream_residency<16, 3>(cus);
        default: *cus = 0; return 0;
    }
}

hipError_t launch_q4k_group(const GroupArgs &g, int total_workgroups, int max_nb, hipStream_t s) {
    constexpr int W = kQ4kWavesLarge;
    const size_t lds = q4k_lds_bytes<W>(1, max_nb);
    hipLaunchKernelGGL((q4k_group_kernel<W>), dim3((unsigned)total_workgroups), dim3(W * 64), lds, s,
                       g);
    return hipGetLastError();
}

}  // namespace qwg
