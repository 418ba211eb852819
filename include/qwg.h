/*
 * qwg.h - C ABI of libqwg: fused dequantize + matrix-vector products over
 * block-quantized weights on AMD Instinct MI355X (gfx950).
 *
 * Formats (as the pages define them):
 *   Q4_K  "用 Python 重写 picoLM" page, dequantize_q4_K listing: 144-byte
 *         super-block of 256 weights = fp16 d (bytes 0-1), fp16 dmin (2-3),
 *         twelve bytes of packed 6-bit sub-block scales and mins (4-15) and
 *         128 bytes of 4-bit quants (16-143). Weight = d*sc_j*q - dmin*mn_j.
 *   IQ3   iq3_pack.py page, module docstring and decode(): 98-byte grouped
 *         container of 256 weights = 64 grid indices (0-63), eight
 *         little-endian uint32 words (64-95: three+one 7-bit sign groups whose
 *         eighth sign is their parity, 4-bit sub-scale code in bits 28-31) and
 *         fp16 d (96-97). Weight = grid[idx][t%4] * sign * d*(0.5+code)*0.5,
 *         grid magnitudes in weight units.
 *   IQ3_XXS  codebook.py page, format table of its docstring, get_d, get_s,
 *         eff_np and dequant: llama.cpp's own IQ3_XXS block, the same 98 bytes
 *         in another order = fp16 d (0-1), 64 grid indices (2-65), eight
 *         uint32 words (66-97, sub-scale s in bits 28-31). Weight = v * eff with
 *         eff = d*(0.5+s)*0.5 and v = grid[idx][t%4] * sign, the grid being
 *         llama.cpp's table as is (entries 4..62; the iq3_pack container stores
 *         the same scheme with the grid halved).
 *   IQ3_S  codebook.py page (format table, get_s, eff_np, dequant, the IQ3_S
 *         branch of encode): 110 bytes = fp16 d (0-1), the low bytes of 64
 *         nine-bit grid indices (2-65), their ninth bits packed little-endian
 *         (66-73), one sign bit per weight packed little-endian (74-105),
 *         eight 4-bit sub-scales as nibbles, low first (106-109).
 *         Weight = sign * grid[idx][t%4] * d*(1+2s), grid [512][4].
 *   IQ4_XS codebook.py page (format table, get_s, eff_np, dequant): 136 bytes
 *         = fp16 d (0-1), the top two bits of eight 6-bit sub-scales at bits
 *         2ib of the uint16 at 2-3, their low four bits as nibbles (4-7), 256
 *         4-bit codes (8-135: byte 8+16ib+j holds weight j of sub-block ib in
 *         its low nibble and weight j+16 in its high nibble, the IQ4_NL order
 *         of that page's encode). Weight = table[q] * d*(s-32), table [16].
 *
 * Common conventions
 *   - Every pointer argument except `stream` is a DEVICE pointer (HIP memory
 *     visible to the current device). `stream` is a hipStream_t passed as
 *     void*; NULL means the default stream.
 *   - A weight matrix W has n_out rows; each row is n_in/256 consecutive
 *     blocks; rows are contiguous (row r starts at r * qwg_row_bytes(fmt, n_in)).
 *     y = W x, the argument order of picoLM's matmul(out, x, W, n_in, n_out,
 *     type) call in that page's model_forward listing.
 *   - Vectors are contiguous fp32. Batched inputs and outputs are row-major:
 *     X is [batch, n_in], Y is [batch, n_out].
 *   - The caller owns every buffer. Calls only enqueue work on `stream` and
 *     return; the caller synchronizes. Outputs must not alias inputs.
 *   - GEMV/GEMM with few 64-row tiles split the n_in sum across workgroups.
 *     The partial sums then go through a per-(device, stream) workspace
 *     (9 MiB + 17 KiB) that the library allocates on the first such call on
 *     that stream (hipMalloc + hipMemset, synchronous) and keeps until
 *     qwg_workspace_release or the end of the process. This is the one place
 *     where the single-matrix calls allocate and keep state. A first such call
 *     on a stream that is being captured into a graph allocates nothing and
 *     returns QWG_ERR_CAPTURE: reserve the workspace before capture
 *     (qwg_workspace_reserve), or use qwg_gemm_q4k_noalloc. Calls on one
 *     stream share its workspace in stream order; a graph captured on a
 *     stream keeps that stream's workspace, so its replays must not overlap
 *     one another or calls on that stream. Concurrent calls on different
 *     streams never share a workspace. The summation order is fixed by the
 *     shapes, so results are deterministic.
 *   - Short batch-1 calls (at most one 64-row tile per compute unit) whose
 *     rows hold at most 8 (Q4_K: n_in <= 2048) or 24 (IQ3, IQ3_XXS, IQ3_S,
 *     IQ4_XS: n_in <= 6144) blocks take whole rows per workgroup: no split
 *     and no workspace.
 *   - Other short batch-1 Q4_K and IQ3 calls (at most one workgroup per compute
 *     unit) whose rows are split add the partial sums through tagged words:
 *     the last split's workgroup waits for its peers' words, which relies on
 *     all of a launch's workgroups becoming resident (true on a device that
 *     runs nothing else that holds its compute units for long). The wait is
 *     bounded (1 s); if it gives up, the tile's rows are stored as NaN, and
 *     later split calls on that stream's workspace may read words left by the
 *     late workgroups: release the workspace (qwg_workspace_release) after
 *     such a result.
 *   - Errors are reported by the returned status (QWG_* below); the library
 *     never aborts, never throws and writes nothing on a validation error.
 *     Validation happens on the host before any HIP call.
 */
#ifndef QWG_H
#define QWG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define QWG_OK 0
#define QWG_ERR_NULL 1     /* a required pointer is NULL */
#define QWG_ERR_SHAPE 2    /* n_in % 256 != 0, n_in outside [256, QWG_MAX_N_IN], n <= 0, n_out < 1 or too large */
#define QWG_ERR_ALIGN 3    /* a pointer is not aligned as documented for the call */
#define QWG_ERR_BATCH 4    /* batch outside 1..QWG_MAX_BATCH */
#define QWG_ERR_HIP 5      /* the HIP runtime reported an error (launch, allocation) */
#define QWG_ERR_FORMAT 6   /* unknown format id */
#define QWG_ERR_CAPTURE 7  /* the stream is capturing and a call would have to allocate */
#define QWG_ERR_TIMEOUT 8  /* a wait of a layer-chain launch gave up (qwg_chain_status) */
#define QWG_ERR_GRID 9     /* a codebook value is not exactly representable in fp16 */

/* format ids */
#define QWG_FMT_Q4K 0
#define QWG_FMT_IQ3 1
#define QWG_FMT_IQ3_XXS 2   /* IQ3 blocks in llama.cpp's byte order */
#define QWG_FMT_IQ3_S 3
#define QWG_FMT_IQ4_XS 4

#define QWG_QK 256
#define QWG_Q4K_BLOCK_BYTES 144
#define QWG_IQ3_BLOCK_BYTES 98
#define QWG_IQ3S_BLOCK_BYTES 110
#define QWG_IQ4XS_BLOCK_BYTES 136
#define QWG_MAX_N_IN 65536          /* 256 super-blocks per row */
#define QWG_MAX_N_OUT (1 << 24)
#define QWG_MAX_BATCH 8
#define QWG_MAX_GROUP 65536         /* GEMVs per grouped launch */

/* Library version (major*10000 + minor*100 + patch). */
int qwg_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char *qwg_strerror(int status);

/* Bytes per row of `n_in` weights in format `fmt` ((n_in/256) * {144, 98, 98,
 * 110, 136}), or -QWG_ERR_SHAPE / -QWG_ERR_FORMAT. */
int64_t qwg_row_bytes(int fmt, int64_t n_in);

/*
 * How a GEMV/GEMM of this shape is decomposed (introspection for tests and
 * tuning): the number of workgroups that share each 64-row tile by splitting
 * the n_in sum (1 = no split), or a negative status for invalid sizes. For
 * Q4_K the plan of the short-call kernels depends on the current device's
 * compute-unit count; with no device the vector engine's plan is returned.
 */
int qwg_plan_splits(int fmt, int64_t n_in, int64_t n_out);

/*
 * Split-sum workspace of `stream` on the current device (see the conventions
 * above). qwg_workspace_reserve creates it now if it does not exist yet
 * (synchronous; QWG_ERR_CAPTURE while the stream is being captured), so that
 * later calls on the stream, including calls recorded into a graph, allocate
 * nothing. qwg_workspace_release frees it (hipFree waits for the device);
 * no work that uses it, and no graph captured with it, may run afterwards.
 * Releasing a stream that has none is a no-op (QWG_OK).
 */
int qwg_workspace_reserve(void *stream);
int qwg_workspace_release(void *stream);

/*
 * Q4_K dequantization ("用 Python 重写 picoLM", dequantize_q4_K listing).
 * src: n/256 consecutive 144-byte blocks, 16-byte aligned.
 * dst: n fp32 weights in block order, 16-byte aligned.
 * n % 256 == 0, n > 0. The result is bit-identical to evaluating, in fp32 with
 * round-to-nearest-even, (d*sc_j)*q - dmin*mn_j per weight.
 */
int qwg_dequant_q4k(const void *src, float *dst, int64_t n, void *stream);

/*
 * IQ3 dequantization (iq3_pack.py page, docstring and decode()).
 * src: n/256 consecutive 98-byte blocks, 2-byte aligned.
 * grid: [256][4] fp32 magnitudes in weight units, 16-byte aligned.
 * dst: n fp32 weights, 16-byte aligned. n % 256 == 0, n > 0.
 * Bit-identical to grid[idx][t%4] * sign * (d*(0.5+code)*0.5) rounded to fp32.
 */
int qwg_dequant_iq3(const void *src, const float *grid, float *dst, int64_t n, void *stream);

/*
 * IQ3_XXS dequantization in llama.cpp's byte order (codebook.py page: format
 * table, get_d, get_s, eff_np, dequant). Arguments, alignment and errors as
 * qwg_dequant_iq3; grid is the codebook in the caller's units (llama.cpp's
 * table: entries 4..62). Bit-identical to (sign * grid[idx][t%4]) *
 * ((d*(0.5+s))*0.5) rounded to fp32 (the scale factor is exact in fp32).
 */
int qwg_dequant_iq3_xxs(const void *src, const float *grid, float *dst, int64_t n,
                        void *stream);

/*
 * y[r] = sum_k W[r,k] x[k] for Q4_K weights (the fused dequantize-and-dot of
 * picoLM's matmul for quantized rows).
 * w: n_out rows of n_in/256 Q4_K blocks, 16-byte aligned.
 * x: n_in fp32, 16-byte aligned.   y: n_out fp32, 4-byte aligned.
 * 256 <= n_in <= QWG_MAX_N_IN, n_in % 256 == 0, 1 <= n_out <= QWG_MAX_N_OUT.
 * Accuracy: |y - exact| <= 2e-6 * sum_k |W[r,k] x[k]| per row for inputs of
 * ordinary magnitude; summation in fp32 in a fixed order.
 */
int qwg_gemv_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                 void *stream);

/*
 * y = W x for IQ3 weights (the fused decode-and-dot of the iq3_pack.py page's
 * decode() followed by the product).
 * w: n_out rows of n_in/256 IQ3 blocks, 2-byte aligned (98-byte blocks put odd
 * blocks at 2 mod 4). The kernel reads whole 16-byte-aligned granules of w but
 * never one that reaches outside [w, w + n_out*row_bytes).
 * grid: [256][4] fp32 magnitudes, 16-byte aligned; every magnitude must be
 * exactly representable in fp16 (true for the integer magnitudes IQ3 grids
 * use): the kernels keep the grid in fp16, and if a value is not exact they
 * store NaN in every output row of the call (the call itself cannot report it:
 * it only enqueues). Group creation checks the grid on the host and returns
 * QWG_ERR_GRID instead.
 * x: n_in fp32, 16-byte aligned. y: n_out fp32, 4-byte aligned.
 * Shape limits and accuracy as qwg_gemv_q4k.
 */
int qwg_gemv_iq3(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                 int64_t n_out, void *stream);

/*
 * y = W x for IQ3_XXS weights in llama.cpp's byte order (codebook.py page, as
 * qwg_dequant_iq3_xxs). Arguments, alignment, the fp16-exact grid requirement,
 * the reads of w, shape limits and accuracy as qwg_gemv_iq3.
 */
int qwg_gemv_iq3_xxs(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                     int64_t n_out, void *stream);

/*
 * IQ3 container encoder (iq3_pack.py page, encode()): fp32 weights x
 * [n_rows][n_in] (finite; n_in % 256 == 0; 4-byte aligned) -> n_rows rows of
 * n_in/256 98-byte blocks at dst (no alignment needed), with the grid [256][4]
 * in weight units (16-byte aligned). Per 256-weight super-block: the parity
 * fix (in each group of eight whose signs multiply to -1, the sign of the
 * first smallest magnitude flips), d = fp16(sqrt(mean(x^2))/20 + 1e-12), and
 * per 32-weight sub-block the code 0..15 and grid rows of least squared error
 * (rows by the least g2 - 2 q.g, q = magnitudes / max(db, 1e-20)). Every step
 * is float32 in a fixed order (numpy's pairwise sums for the mean and the
 * errors, q.g summed left to right without fused multiply-adds, first minimum
 * on ties), so the bytes are reproducible and match the CPU reference.
 */
int qwg_encode_iq3(void *dst, const float *x, const float *grid, int64_t n_rows, int64_t n_in,
                   void *stream);

/*
 * IQ3_S and IQ4_XS (codebook.py page; layouts above).
 * qwg_dequant_iq3s: src n/256 blocks of 110 bytes (2-byte aligned), grid
 * [512][4] fp32 (16-byte aligned), dst n fp32 (16-byte aligned).
 * qwg_dequant_iq4xs: src n/256 blocks of 136 bytes (4-byte aligned), table
 * [16] fp32 (16-byte aligned), dst as above.
 * Both bit-identical to (sign * entry) * eff rounded to fp32, eff exact.
 *
 * qwg_gemv_iq3s / qwg_gemv_iq4xs: y = W x on row-major blocks as a file stores
 * them (n_out rows of n_in/256 blocks, rows back to back; w 16-byte aligned,
 * the row length need not be a multiple of 16 bytes), x 16-byte aligned, y
 * 4-byte aligned, the grid/table 16-byte aligned. Each 64-row tile's blocks
 * are copied to LDS 16-byte granule by granule and read at their offsets; no
 * byte outside w's n_out*row_bytes is read.
 *
 * The same GEMVs also run on a tile layout made once at load time:
 * qwg_pack_iq3s_tiles / qwg_pack_iq4xs_tiles take row-major blocks (src
 * 2-byte aligned, n_out rows of n_in/256 blocks) and write
 * qwg_tiled_bytes(fmt, n_in, n_out) bytes (dst 16-byte aligned): for each
 * 64-row tile and block column, the 64 rows' blocks regrouped by field (IQ3_S:
 * index bytes [G][row][16], sign bytes [G][row][8], ninth-bit bytes
 * [G][row][2], sub-scale bytes [row][4], d [row][2]; IQ4_XS: code bytes
 * [G][row][32], bytes 0-7 [row][8]; G = 0..3 is the pair of sub-blocks 2G,
 * 2G+1); rows past n_out are zero blocks. Every byte of every block is kept.
 * qwg_gemv_iq3s_tiled / qwg_gemv_iq4xs_tiled: y = W x on that layout (w
 * 16-byte aligned; x, y, grid/table as above).
 * For all four GEMVs every grid or table value must be exactly representable
 * in fp16 (true for the integer values of these codebooks); otherwise every
 * output row of the call is NaN (group creation returns QWG_ERR_GRID).
 * Shape limits and accuracy as qwg_gemv_q4k.
 */
int qwg_dequant_iq3s(const void *src, const float *grid, float *dst, int64_t n, void *stream);
int qwg_dequant_iq4xs(const void *src, const float *table, float *dst, int64_t n, void *stream);
int qwg_pack_iq3s_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream);
int qwg_pack_iq4xs_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream);
int qwg_gemv_iq3s(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                  int64_t n_out, void *stream);
int qwg_gemv_iq4xs(float *y, const float *x, const void *w, const float *table, int64_t n_in,
                   int64_t n_out, void *stream);
int qwg_gemv_iq3s_tiled(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                        int64_t n_out, void *stream);
int qwg_gemv_iq4xs_tiled(float *y, const float *x, const void *w, const float *table,
                         int64_t n_in, int64_t n_out, void *stream);

/*
 * qwg_gemv_iq3 with an explicit work decomposition (tuning and testing):
 * `waves` wavefronts per workgroup (4, 8 or 16; 0 = automatic) and `splits`
 * workgroups sharing each 64-row tile's n_in sum (1..n_in/256; 0 = automatic).
 * Same bound for every choice. QWG_ERR_SHAPE for an unsupported choice (also
 * when splits*ceil(n_out/64)*64 partial sums exceed the split workspace, or
 * ceil(n_out/64) > 4096 with splits > 1).
 */
int qwg_gemv_iq3_ex(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                    int64_t n_out, int waves, int splits, void *stream);

/*
 * Y[b, r] = sum_k W[r,k] X[b,k] for 1 <= batch <= QWG_MAX_BATCH, Q4_K weights:
 * every weight is decoded once and applied to all `batch` activation rows.
 * x: [batch, n_in] fp32 row-major, 16-byte aligned. y: [batch, n_out] fp32
 * row-major, 4-byte aligned. batch == 1 computes the same as qwg_gemv_q4k.
 * batch >= 2 runs on the matrix cores (bf16 MFMA with the activations split
 * exactly into three bf16 parts and the quants entered as exact integers; only
 * the fp32 accumulation rounds), within the same bound.
 */
int qwg_gemm_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                 int batch, void *stream);

/*
 * qwg_gemm_q4k for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, kernels, work decomposition and results (bit-identical to
 * qwg_gemm_q4k), but split sums go through a fixed scratch array that the
 * library's code object holds on every GPU (1 MiB of partial sums, 1 MiB of
 * tagged split words, 4096 tile counters and 256 tile epochs, held until the
 * process ends) instead of the per-stream workspace, so no call allocates or
 * frees anything. The first call on a device also enqueues a small kernel
 * that zeroes everything but the partial sums. Every shape
 * the plans produce fits; a plan that did not fit the scratch would return
 * QWG_ERR_SHAPE. All calls on one GPU share the one scratch array: calls that
 * overlap in time on that GPU (on different streams, or replays of graphs
 * that contain such calls) race and must not be made.
 */
int qwg_gemm_q4k_noalloc(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                         int batch, void *stream);

/*
 * qwg_gemm_q4k with an explicit work decomposition (tuning and testing):
 * `waves` selects the engine: 4, 8 or 16 wavefronts per 64-row tile on the
 * vector ALUs; 1 or 2 = the matrix-core pipeline (batch >= 2 only), one
 * workgroup per (tile, split) taking one super-block column per stage with 4
 * wavefronts, or two columns with 8; 3 = the persistent matrix-core stream
 * (batch >= 2 only: resident workgroups walk the (tile, split) items with a
 * ring of stages that runs ahead across them); 0 = automatic among these
 * engines (the persistent stream for batch >= 2; qwg_gemm_q4k itself runs a
 * batch-1 matrix of up to 256 tiles on the short-call kernels instead); `splits`
 * workgroups sharing each tile's n_in sum (1..n_in/256; 0 = automatic). The
 * result satisfies the same bound for every choice; the summation order (so
 * the rounding) depends on it. Returns QWG_ERR_SHAPE for an unsupported
 * choice (also when splits*batch*ceil(n_out/64)*64 partial sums exceed the
 * split workspace of 2*2048*8*64 floats, or ceil(n_out/64) > 4096 with splits > 1).
 */
int qwg_gemm_q4k_ex(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                    int batch, int waves, int splits, void *stream);

/*
 * Tile layout for Q4_K (a one-time, load-time reordering of the same 144-byte
 * blocks for the GEMV's streaming pattern): for each 64-row tile, for each
 * block column b, the tile's 64 blocks of column b back to back (9216 bytes);
 * rows past n_out in the last tile are zero blocks. Block (r, b) of the
 * row-major matrix moves to byte ((r/64)*(n_in/256) + b)*9216 + (r%64)*144.
 * A stage of the GEMV then copies one contiguous 9216-byte run instead of 64
 * rows' 144-byte pieces.
 *
 * Tile layout for IQ3 (102 bytes per block): the same tile and column order
 * (column (t, b) at (t*(n_in/256) + b)*6528), each 6528-byte column regrouped
 * by field so that every read of the GEMV is aligned and conflict-free: the 64
 * rows' index bytes 16G..16G+15 for G = 0..3 ([G][row][16], 4096 bytes); the
 * sign groups of their words 2G, 2G+1 as sign bytes ([G][row][8], 2048 bytes:
 * byte k of a word's four is its group k's seven stored signs with, in bit 7,
 * the eighth that the even-count rule implies); the words' 4-bit scales
 * ([G][row], 256 bytes: word 2G's in the low nibble, 2G+1's in the high one);
 * then their d ([row][2], 128 bytes). Every stored bit of every block is kept;
 * the implied signs are written out so that the GEMV need not recover them.
 *
 * qwg_tiled_bytes: bytes of the tile layout (ceil(n_out/64)*64 rows) for
 * any QWG_FMT_* format, or a negative status.
 * qwg_pack_q4k_tiles: src (row-major, as qwg_gemv_q4k takes it) -> dst (tile
 * layout, qwg_tiled_bytes bytes); both 16-byte aligned, must not overlap.
 * qwg_gemv_q4k_tiled: qwg_gemv_q4k on tile-layout weights (same arguments,
 * alignment and accuracy).
 * qwg_gemm_q4k_tiled: qwg_gemm_q4k on tile-layout weights (same arguments,
 * alignment and accuracy; batch 1 is qwg_gemv_q4k_tiled). For batch >= 2 the
 * result is bit-identical to qwg_gemm_q4k on the row-major weights.
 * qwg_pack_iq3_tiles: as qwg_pack_q4k_tiles for IQ3 (src 2-byte aligned, dst
 * 16-byte aligned).
 * qwg_gemv_iq3_tiled: qwg_gemv_iq3 on tile-layout weights (w 16-byte aligned;
 * otherwise the same arguments and accuracy).
 * qwg_pack_iq3_xxs_tiles: as qwg_pack_iq3_tiles for row-major IQ3_XXS blocks
 * in llama.cpp's order; the result is the same IQ3 tile layout (each field
 * moved to its place), so qwg_gemv_iq3_tiled and the tiled IQ3 groups take
 * it, with llama.cpp's grid.
 */
int64_t qwg_tiled_bytes(int fmt, int64_t n_in, int64_t n_out);
int qwg_pack_q4k_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream);
int qwg_gemm_q4k_tiled(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                       int batch, void *stream);
int qwg_gemv_q4k_tiled(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                       void *stream);
int qwg_pack_iq3_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream);
int qwg_gemv_iq3_tiled(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                       int64_t n_out, void *stream);
int qwg_pack_iq3_xxs_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out,
                           void *stream);

/*
 * Grouped GEMV: many independent GEMVs of one format in one launch (one grid
 * whose workgroups belong to different matrices), for streams of independent
 * weight-bound products such as the q/k/v or gate/up projections that share an
 * activation vector, or a whole decode step's weight stream when its inputs are
 * independent. Same math and accuracy as qwg_gemv_q4k / qwg_gemv_iq3 for every
 * member.
 *
 * qwg_gemv_desc: one member, fields as the qwg_gemv_q4k / qwg_gemv_iq3
 * arguments (device pointers, same alignment and shape rules).
 * qwg_group_create_q4k / qwg_group_create_iq3: validate every member (the
 * first failing member's status is returned, nothing is allocated) and, for
 * the codebook formats, copy the grid or table to the host and check that
 * every value is exactly representable in fp16 (QWG_ERR_GRID otherwise), then
 * copy the launch plan to a device buffer owned by the group (hipMalloc +
 * hipMemcpy: synchronous). `descs` is a host array of `count` members
 * (1..QWG_MAX_GROUP) and is not kept. The member pointers (and the IQ3 grid,
 * shared by all members, rules as for qwg_gemv_iq3) are baked into the plan:
 * reuse the same buffers (e.g. fixed activation/output buffers of a decode
 * loop) on every run. A group with fewer 64-row tiles than the workgroups the
 * device holds at once (a few layers' projections rather than a whole decode
 * step) splits its members' n_in sums across workgroups; the partial sums
 * and tile counters then live in the group's device buffer (the counters are
 * zeroed at creation and every run leaves them at zero), so runs of one such
 * group must not overlap in time (e.g. on two streams): they would race.
 * qwg_group_run: enqueues the whole group on `stream` (asynchronous).
 * qwg_group_workgroups: number of 64-row tiles of one run, or a negative
 * status.
 * qwg_group_destroy: frees the plan (hipFree: synchronous; no run of the group
 * may be pending). NULL is accepted.
 */
typedef struct qwg_gemv_desc {
    float *y;
    const float *x;
    const void *w;
    int64_t n_in;
    int64_t n_out;
} qwg_gemv_desc;

typedef struct qwg_group qwg_group;

int qwg_group_create_q4k(const qwg_gemv_desc *descs, int count, qwg_group **group);
int qwg_group_create_iq3(const qwg_gemv_desc *descs, int count, const float *grid,
                         qwg_group **group);
/* As qwg_group_create_q4k / _iq3, every member's weights in the tile layout
 * (16-byte aligned). */
int qwg_group_create_q4k_tiled(const qwg_gemv_desc *descs, int count, qwg_group **group);
/*
 * Batched group: Y_i[b, r] = sum_k W_i[r, k] X_i[b, k] for every member i and
 * 2 <= batch <= QWG_MAX_BATCH activation rows, one launch per run (e.g. every
 * projection of a decoding step for `batch` sequences at once). Each member's
 * x points at [batch][n_in] fp32 row-major (16-byte aligned) and y at
 * [batch][n_out] fp32 row-major (4-byte aligned); w holds row-major Q4_K
 * blocks (16-byte aligned). The matrix-core engine of qwg_gemm_q4k runs one
 * workgroup per 64-row tile of every member (no split sums), within the same
 * bound as qwg_gemm_q4k. Returns QWG_ERR_BATCH for a batch outside 2..8;
 * otherwise as qwg_group_create_q4k. Runs may overlap (no shared scratch).
 */
int qwg_group_create_q4k_batched(const qwg_gemv_desc *descs, int count, int batch,
                                 qwg_group **group);
/* As qwg_group_create_q4k_batched, every member's weights in the tile layout
 * (qwg_pack_q4k_tiles, 16-byte aligned): each pipeline stage is one contiguous
 * 9216-byte run. Bit-identical to the row-major group on the same weights. */
int qwg_group_create_q4k_batched_tiled(const qwg_gemv_desc *descs, int count, int batch,
                                       qwg_group **group);
int qwg_group_create_iq3_tiled(const qwg_gemv_desc *descs, int count, const float *grid,
                               qwg_group **group);
/* Groups of IQ3_S (grid [512][4]) or IQ4_XS (table [16]) members, on
 * row-major blocks (every member's w 16-byte aligned, as for qwg_gemv_iq3s) or
 * in the tile layout (_tiled), rules as for the IQ3 groups; the grid/table is
 * shared by all members. */
int qwg_group_create_iq3s(const qwg_gemv_desc *descs, int count, const float *grid,
                          qwg_group **group);
int qwg_group_create_iq4xs(const qwg_gemv_desc *descs, int count, const float *table,
                           qwg_group **group);
int qwg_group_create_iq3s_tiled(const qwg_gemv_desc *descs, int count, const float *grid,
                                qwg_group **group);
int qwg_group_create_iq4xs_tiled(const qwg_gemv_desc *descs, int count, const float *table,
                                 qwg_group **group);
int qwg_group_run(const qwg_group *group, void *stream);
int qwg_group_workgroups(const qwg_group *group);
int qwg_group_destroy(qwg_group *group);

/*
 * Layer chain: a decoder's per-token weight stream as one launch whose phases
 * run in dependency order ("用 Python 重写 picoLM" page, model_forward and
 * forward listings: per layer the q/k/v products read the normalized x, the
 * output projection reads the attention output, gate/up read the normalized
 * residual, down reads the SwiGLU activation, the next layer reads the updated
 * x, the LM head reads the final norm). The operations between the products
 * (norms, attention, activation) are outside this library, so the launch
 * treats each phase as depending on all outputs of the phase before it: no
 * product of phase p+1 reads its activations before every member of phase p
 * has stored its result. Weights do not depend on activations and are
 * fetched ahead across phases.
 *
 * How the phases wait (chosen at creation): tagged, when every x that
 * overlaps a y of the chain lies wholly inside the y of one member of an
 * earlier phase, no two members' y overlap and no y overlaps the x of a member
 * of an earlier phase (nothing is overwritten that an earlier phase reads):
 * the unit that finishes a tile of a phase stores a tagged done word (8
 * bytes: the tile's sum of squares of y, and the run's tag for that phase),
 * a member whose y a later member reads also stores its rows as tagged
 * 8-byte words, and a phase waits until it has loaded the done words of every
 * tile of the phase before it with this run's tag, reading activations made
 * by the chain as tagged words. Otherwise (or with QWG_CHAIN_TAGGED=0 in the
 * environment at creation) every workgroup publishes a flag per phase and
 * polls all flags before a dependent phase. Both give the same results.
 *
 * qwg_chain_create_q4k: `count` members (qwg_gemv_desc, Q4_K weights in the
 * tile layout of qwg_pack_q4k_tiles, 16-byte aligned; x 16-byte aligned, y
 * 4-byte aligned; shape rules as qwg_gemv_q4k) in phase order: the first
 * phase_sizes[0] members form phase 0, the next phase_sizes[1] phase 1, and so
 * on (n_phases >= 1, every size >= 1, the sizes summing to count). A member's
 * x may be (or overlap) the y of a member of an earlier phase: it is then read
 * only after that phase has completed. QWG_ERR_SHAPE if an x overlaps a y of
 * the same phase. Validation happens before anything is allocated; then the
 * plan (one workgroup per compute unit, each phase's work spread over all of
 * them) is copied to a device buffer owned by the chain (hipMalloc + hipMemcpy:
 * synchronous). The member pointers are baked into the plan; reuse the same
 * buffers on every run (e.g. fixed activation/output buffers of a decode loop).
 * qwg_chain_run: enqueues the whole chain on `stream` (asynchronous). The
 * launch holds one workgroup on every compute unit and its phases wait for one
 * another, so it needs the whole device: run nothing else on the device at the
 * same time, and do not overlap two runs of one chain. Every wait is bounded
 * (0.2 s): a wait that gives up marks the chain's error word and the launch
 * ends early (outputs then undefined).
 * qwg_chain_status: waits for the device (hipDeviceSynchronize), then returns
 * QWG_OK, or QWG_ERR_TIMEOUT if a wait of an earlier run gave up (the chain is
 * re-armed and can run again).
 * qwg_chain_phases: number of phases of one launch (a phase with more work
 * than the device's compute units take at once runs as several), or a negative
 * status.
 * qwg_chain_tagged: 1 if the phases wait on tagged done words, 0 if on flags,
 * or a negative status.
 * qwg_chain_destroy: frees the plan (hipFree: synchronous). NULL is accepted.
 * Results meet the same bound as qwg_gemv_q4k for every member and are
 * bitwise reproducible (fixed summation order).
 */
typedef struct qwg_chain qwg_chain;

int qwg_chain_create_q4k(const qwg_gemv_desc *descs, int count, const int *phase_sizes,
                         int n_phases, qwg_chain **chain);
int qwg_chain_run(const qwg_chain *chain, void *stream);
int qwg_chain_status(qwg_chain *chain);
int qwg_chain_phases(const qwg_chain *chain);
int qwg_chain_tagged(const qwg_chain *chain);
int qwg_chain_destroy(qwg_chain *chain);

#ifdef __cplusplus
}
#endif
#endif
