// Short single GEMV calls for gfx950 (batch 1, a few MB of weights).
//
// Format and product: "用 Python 重写 picoLM" page, dequantize_q4_K and matmul
// listings (y = W x over 144-byte Q4_K super-blocks).
//
// A call of a few MB is latency-bound. Measured on MI355X (kernel trace, cold
// weights): an empty kernel takes 1.4 us; a plain read of 2 MB by 256
// workgroups 2.5 us, by 32 workgroups of 64 KB 3.4 us (LDS-DMA as fast as
// loads into registers); the split epilogue of the stream engines (store the
// partials, wait, count at the tile's counter, the last one loads and sums)
// adds 1.6 us at two splits and 3.9 us at eight. And a whole 64-row tile per
// compute unit is slow to compute: its dot products take ~1.3 us of one
// compute unit's vector ALUs, and activations read from LDS as broadcast
// operands cost as much LDS bandwidth as full reads (a first version with 16
// wavefronts per tile and the activations in LDS took 7.4 us for 2048 x 2048).
//
// So the work is spread over (up to) every compute unit: each 64-row tile's
// super-blocks are split over S workgroups (tiles x S <= compute units), and a
// workgroup has eight wavefronts per super-block column it holds (four when it
// holds three or four columns; at most kShortMaxBlocks). Each wavefront
// requests its share of its column's nine 1 KB pieces (LDS-DMA), the
// activations of its sub-block (or quant chunk) as scalar loads (operands
// straight from SGPRs) and one activation per lane of the chunk (for the
// sub-block sums), all before one wait and one barrier; then it computes its
// sub-block (chunk) of the column for the tile's 64 rows (lane = row), and the
// row sums of the workgroup's wavefronts meet in LDS in wavefront order.
// Measured for 2048 x 2048 (256 workgroups of one column): from the kernel's
// start, the data is in LDS after ~1.4 us, a chunk's dot takes 0.5 us, the
// last split's wait for its peers 1.4 us.
//
// Splits end through tagged words (short_dev.h).
#include "qwg_device.h"
#include "q4k_dot.h"
#include "short_dev.h"

namespace qwg {

namespace {

constexpr int kColBytes = kTileRows * kQ4kBytes;                  // 9216
// C columns, then the row sums [W wavefronts][64] fp32
constexpr int lds_bytes(int c, int w) { return c * kColBytes + w * kTileRows * 4; }
static_assert(kColBytes == 9 * 1024, "a column is nine 1 KB copies");

// Sub-block 2G + H of a super-block for this lane's row (quant chunk G's low
// nibbles for H = 0, high nibbles for H = 1), as q4k_chunk_2chains computes
// each of its two halves: the quants enter as fp16 subnormals (low nibbles
// q * 2^-24, high nibbles q * 2^-20, folded back into d*sc), the min term
// takes the sub-block's activation sum sx.
template <int G, int H, typename XAt>
__device__ __forceinline__ void q4k_subblock(const uint8_t *rowp, XAt xat, float sx, uint32_t mask,
                                             float &acc) {
    const uint4 h = *(const uint4 *)rowp;
    const uint4 qa = *(const uint4 *)(rowp + 16 + 32 * G);
    const uint4 qb = *(const uint4 *)(rowp + 32 + 32 * G);
    uint32_t sc0, sc1, mn0, mn1;
    q4k_scales<G>(h, sc0, sc1, mn0, mn1);
    const float dsc = h2f_lo(h.x) * (float)(H ? (sc1 << 20) : (sc0 << 24));
    const float dmn = h2f_hi(h.x) * (float)(H ? mn1 : mn0);
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float s[2] = {0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int c = m & 1;
        const uint32_t e = q[m] & mask;          // bytes 0, 2
        const uint32_t o = (q[m] >> 8) & mask;   // bytes 1, 3
        s[c] = __builtin_fmaf(h2f_lo(e), xat(4 * m + 0), s[c]);
        s[c] = __builtin_fmaf(h2f_lo(o), xat(4 * m + 1), s[c]);
        s[c] = __builtin_fmaf(h2f_hi(e), xat(4 * m + 2), s[c]);
        s[c] = __builtin_fmaf(h2f_hi(o), xat(4 * m + 3), s[c]);
    }
    float r = acc;
    r = __builtin_fmaf(dsc, s[0] + s[1], r);
    r = __builtin_fmaf(-dmn, sx, r);
    acc = r;
}

// C super-block columns per workgroup, 4H wavefronts per column: wavefront w
// takes column w / 4H, quant chunk G = (w / H) % 4 and, for H = 2, one of the
// chunk's two sub-blocks (w % 2).
template <int C, int H>
__global__ __launch_bounds__(256 * C * H) void q4k_short_kernel(GemvArgs a, ShortState st, int tiled) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int WPC = 4 * H;        // wavefronts per column
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = wave / WPC;         // column of the workgroup's range
    const int G = (wave / H) & 3;     // quant chunk
    const int hh = wave % H;          // sub-block of the chunk (H = 2)
    int tile, split;
    if (!short_item(a, tile, split)) return;
    const int kb0 = split * a.nb / a.splits;
    const int kb1 = (split + 1) * a.nb / a.splits;
    const bool live = kb0 + j < kb1;
    const int b = kb0 + j;            // this wavefront's super-block (if live)
    const int row0 = tile * kTileRows;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // Column j's 9216 bytes: copies i, i + WPC, ... of its nine 1 KB pieces,
    // i = wave % WPC (piece q: 16-byte chunk k = 64 q + lane = row k / 9,
    // bytes 16 (k % 9)).
    if (live) {
        for (int q = wave % WPC; q < 9; q += WPC) {
            const int k = 64 * q + lane;
            const uint32_t dst = lds0 + j * kColBytes + 1024 * q;
            if (tiled) {
                dma16(a.w + ((int64_t)tile * a.nb + b) * kColBytes + 16 * k, dst);
            } else {
                const int r = k / 9;
                const int row = min(row0 + r, a.n_out - 1);
                dma16(a.w + (int64_t)row * a.row_bytes + (int64_t)b * kQ4kBytes + 16 * (k - 9 * r), dst);
            }
        }
    }
    // The wavefront's activations (the chunk's 64, or its sub-block's 32) as
    // scalar operands, and one per lane of the chunk for the sub-block sums,
    // requested before the wait so that they arrive with the weights.
    constexpr int NX = 64 / H;
    const int xb = live ? b : kb0;
    const cfloat_p xg = as_scalar(a.x) + (int64_t)kQK * xb + 64 * G + NX * hh;
    float xs[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) xs[i] = xg[i];
    const float xl = a.x[(int64_t)kQK * xb + 64 * G + lane];
    // The tile's epoch (split launches), needed only at the end.
    uint32_t epoch = 0;
    if (a.splits > 1 && wave == 0)
        epoch = __hip_atomic_load(&st.epochs[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();
    lds_barrier();

    float acc = 0.0f;
    if (live) {
        const float hs = half_wave_sum(xl);
        const float sx0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hs), 16));
        const float sx1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hs), 48));
        const uint8_t *rowp = smem + j * kColBytes + lane * kQ4kBytes;
        auto xat = [&](int i) { return xs[i]; };
        if constexpr (H == 1) {
            const uint32_t mlo = opaque(0x000F000Fu);
            const uint32_t mhi = opaque(0x00F000F0u);
            switch (G) {
                case 0: q4k_chunk_2chains<0>(rowp, xat, sx0, sx1, mlo, mhi, acc); break;
                case 1: q4k_chunk_2chains<1>(rowp, xat, sx0, sx1, mlo, mhi, acc); break;
                case 2: q4k_chunk_2chains<2>(rowp, xat, sx0, sx1, mlo, mhi, acc); break;
                default: q4k_chunk_2chains<3>(rowp, xat, sx0, sx1, mlo, mhi, acc); break;
            }
        } else if (hh == 0) {
            const uint32_t m = opaque(0x000F000Fu);
            switch (G) {
                case 0: q4k_subblock<0, 0>(rowp, xat, sx0, m, acc); break;
                case 1: q4k_subblock<1, 0>(rowp, xat, sx0, m, acc); break;
                case 2: q4k_subblock<2, 0>(rowp, xat, sx0, m, acc); break;
                default: q4k_subblock<3, 0>(rowp, xat, sx0, m, acc); break;
            }
        } else {
            const uint32_t m = opaque(0x00F000F0u);
            switch (G) {
                case 0: q4k_subblock<0, 1>(rowp, xat, sx1, m, acc); break;
                case 1: q4k_subblock<1, 1>(rowp, xat, sx1, m, acc); break;
                case 2: q4k_subblock<2, 1>(rowp, xat, sx1, m, acc); break;
                default: q4k_subblock<3, 1>(rowp, xat, sx1, m, acc); break;
            }
        }
    }
    float *red = (float *)(smem + C * kColBytes);
    red[wave * 64 + lane] = acc;
    lds_barrier();
    if (wave != 0) return;
    float total = red[lane];
    for (int w = 1; w < WPC * C; ++w) total += red[w * 64 + lane];
    short_epilogue(a, st, tile, split, epoch, total);
}

// Row-group kernel (rows of at most eight super-blocks): a workgroup takes
// kRgRows = 8 whole rows, so no split sums meet through memory. Eight
// wavefronts: wavefront j takes sub-block j of every super-block (quant chunk
// j / 2, low nibbles for even j); lane r + 8s takes row r of the group and
// super-block s. The group's rows (8 x nb x 144 bytes) are copied into LDS;
// each lane loads the 32 activations of its sub-block into registers (eight
// 16-byte loads; the wavefront's lanes read eight distinct 128-byte pieces,
// which is what limits this mapping to short rows: at 22 super-blocks per row
// a split tile with scalar activations measured faster, 7.8 against 8.2 us per
// call, and 5.96 against 6.62 us of kernel time for block sets of four chunk
// wavefronts). A lane's sum meets its row's other super-blocks across the
// wavefront (xor shuffles over lanes r + 8s), the eight wavefronts' in LDS in
// wavefront order. Measured against the split short-call kernel (kernel
// trace, cold weights): 2048 x 2048 4.72 -> 4.24 us, 5632 x 2048 6.16 -> 5.80
// us, 256 x 2048 4.08 either way; event time per call, alternating runs on one
// box: 6.56 -> 6.04, 7.92 -> 7.36, 6.24-6.4 -> 6.12-6.16 us.
constexpr int kRgRows = 8;
constexpr int kRgWaves = 8;
constexpr int kRgMaxBlocks = 8;
constexpr int rg_lds_bytes(int nb) {
    return ((kRgRows * nb * 9 + 63) / 64) * 1024 + kRgWaves * kRgRows * 4;
}

__global__ __launch_bounds__(64 * kRgWaves) void q4k_rows_kernel(GemvArgs a, int tiled) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int R = kRgRows;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = wave >> 1;
    const int hh = wave & 1;
    const int row0 = blockIdx.x * R;
    const int nb = a.nb;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    // Copy: 16-byte chunk k of the group, as 64-chunk instructions; the last
    // instruction's lanes past the end re-read the last chunk into LDS past
    // the group's bytes (rg_lds_bytes rounds up to whole instructions).
    const int nchunks = R * nb * 9;
    for (int k0 = 64 * wave; k0 < nchunks; k0 += 64 * kRgWaves) {
        const int k = min(k0 + lane, nchunks - 1);
        if (tiled) {
            // block b of the group's rows: R x 144 contiguous bytes of the
            // tile column (the last tile is padded to 64 rows); LDS [b][r][144]
            const int b = k / (R * 9);
            dma16(a.w + ((int64_t)(row0 >> 6) * nb + b) * kColBytes + (row0 & 63) * kQ4kBytes +
                      16 * (k - b * R * 9),
                  lds0 + 16 * k0);
        } else {
            // row r: nb x 144 contiguous bytes (rows past n_out re-read the
            // last row); LDS [r][b][144]
            const int r = k / (nb * 9);
            const int row = min(row0 + r, a.n_out - 1);
            dma16(a.w + (int64_t)row * a.row_bytes + 16 * (k - r * nb * 9), lds0 + 16 * k0);
        }
    }
    const int r = lane & (R - 1);
    const int b = lane >> 3;
    const bool live = b < nb;
    f32x4 xv[8];
    {
        const f32x4 *xp = (const f32x4 *)(a.x + (int64_t)kQK * min(b, nb - 1) + 32 * wave);
#pragma unroll
        for (int q = 0; q < 8; ++q) xv[q] = xp[q];
    }
    wait_vmcnt<0>();
    lds_barrier();

    float acc = 0.0f;
    if (live) {
        const uint8_t *rowp = smem + (tiled ? (b * R + r) : (r * nb + b)) * kQ4kBytes;
        float t[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = (xv[q][0] + xv[q][1]) + (xv[q][2] + xv[q][3]);
        const float sx = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
        auto xat = [&](int e) { return xv[e >> 2][e & 3]; };
        const uint32_t m = opaque(hh ? 0x00F000F0u : 0x000F000Fu);
        if (hh == 0) {
            switch (G) {
                case 0: q4k_subblock<0, 0>(rowp, xat, sx, m, acc); break;
                case 1: q4k_subblock<1, 0>(rowp, xat, sx, m, acc); break;
                case 2: q4k_subblock<2, 0>(rowp, xat, sx, m, acc); break;
                default: q4k_subblock<3, 0>(rowp, xat, sx, m, acc); break;
            }
        } else {
            switch (G) {
                case 0: q4k_subblock<0, 1>(rowp, xat, sx, m, acc); break;
                case 1: q4k_subblock<1, 1>(rowp, xat, sx, m, acc); break;
                case 2: q4k_subblock<2, 1>(rowp, xat, sx, m, acc); break;
                default: q4k_subblock<3, 1>(rowp, xat, sx, m, acc); break;
            }
        }
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    float *red = (float *)(smem + rg_lds_bytes(nb) - kRgWaves * R * 4);
    if (lane < R) red[wave * R + lane] = acc;
    lds_barrier();
    if (wave != 0 || lane >= R) return;
    float total = red[lane];
#pragma unroll
    for (int w = 1; w < kRgWaves; ++w) total += red[w * R + lane];
    if (row0 + lane < a.n_out) a.y[row0 + lane] = total;
}

}  // namespace

bool q4k_rows_fits(int nb) { return nb <= kRgMaxBlocks; }

hipError_t launch_q4k_rows(const GemvArgs &a, bool tiled, hipStream_t s) {
    if (a.nb > kRgMaxBlocks) return hipErrorInvalidValue;
    const dim3 grid((a.n_out + kRgRows - 1) / kRgRows);
    hipLaunchKernelGGL(q4k_rows_kernel, grid, dim3(64 * kRgWaves), rg_lds_bytes(a.nb), s, a,
                       tiled ? 1 : 0);
    return hipGetLastError();
}

int short_plan_splits(int tiles, int nb, int cus) {
    if (tiles > kShortMaxTiles || tiles > cus) return 0;
    int sp = cus / tiles;
    if (sp > nb) sp = nb;
    if (sp > kShortMaxSplits) sp = kShortMaxSplits;
    return (nb + sp - 1) / sp <= kShortMaxBlocks ? sp : 0;
}

hipError_t launch_q4k_short(const GemvArgs &a, const ShortState &st, bool tiled, hipStream_t s) {
    const int cols = (a.nb + a.splits - 1) / a.splits;   // most columns of one split
    const dim3 grid(short_grid(a.tiles, a.splits));
    const int t = tiled ? 1 : 0;
    if (cols == 1)
        hipLaunchKernelGGL((q4k_short_kernel<1, 2>), grid, dim3(512), lds_bytes(1, 8), s, a, st, t);
    else if (cols == 2)
        hipLaunchKernelGGL((q4k_short_kernel<2, 2>), grid, dim3(1024), lds_bytes(2, 16), s, a, st, t);
    else
        hipLaunchKernelGGL((q4k_short_kernel<4, 1>), grid, dim3(1024), lds_bytes(4, 16), s, a, st, t);
    return hipGetLastError();
}

}  // namespace qwg
