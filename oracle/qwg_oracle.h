/*
 * qwg oracle: plain, slow CPU reference for the quantized-weight decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load, call or link this code. It shares no
 * source, header, table or helper with the HIP library, and the library never
 * calls it.
 *
 * Formats follow the pages' definitions:
 *   Q4_K  - "用 Python 重写 picoLM" (rewriting picoLM in Python), the
 *           dequantize_q4_K listing: 144-byte super-block of 256 weights.
 *   IQ3   - the iq3_pack.py page, module docstring (layout) and decode():
 *           98-byte grouped container of 256 weights.
 *   IQ3_XXS - the codebook.py page (format table, get_d, get_s, eff_np,
 *           dequant): the same 98 bytes in llama.cpp's order (d first).
 *   IQ3_S, IQ4_XS - the codebook.py page (format table, get_s, eff_np,
 *           dequant, and the IQ3_S branch of encode): 110 and 136 bytes.
 *
 * Every entry point returns 0 on success, 2 when a size is invalid
 * (n % 256 != 0, n < 0, n_out < 1, batch outside 1..8), 1 on a NULL pointer.
 */
#ifndef QWG_ORACLE_H
#define QWG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_QK 256          /* weights per super-block (both formats) */
#define ORC_Q4K_BYTES 144   /* 2 + 2 + 12 + 128 */
#define ORC_IQ3_BYTES 98    /* 64 + 32 + 2 */
#define ORC_IQ3S_BYTES 110  /* 2 + 64 + 8 + 32 + 4 */
#define ORC_IQ4XS_BYTES 136 /* 2 + 2 + 4 + 128 */

/* IEEE 754 binary16 -> binary32, exact (subnormals, infinities, NaN). */
float orc_f16_to_f32(uint16_t h);
/* binary32 -> binary16 bits, round to nearest even. */
uint16_t orc_f32_to_f16(float f);

/* The 12-byte packed 6-bit scale/min field of a Q4_K block <-> sc[8], mn[8]. */
void orc_q4k_unpack_scales(const uint8_t p[12], uint8_t sc[8], uint8_t mn[8]);
void orc_q4k_pack_scales(const uint8_t sc[8], const uint8_t mn[8], uint8_t p[12]);

/* Decode n weights (n % 256 == 0) from n/256 consecutive blocks into fp32. */
int orc_dequant_q4k(const uint8_t *src, int64_t n, float *dst);
int orc_dequant_iq3(const uint8_t *src, const float *grid, int64_t n, float *dst);
int orc_dequant_iq3_xxs(const uint8_t *src, const float *grid, int64_t n, float *dst);
/* grid: [512][4] fp32; table: [16] fp32 */
int orc_dequant_iq3s(const uint8_t *src, const float *grid, int64_t n, float *dst);
int orc_dequant_iq4xs(const uint8_t *src, const float *table, int64_t n, float *dst);

/*
 * y[n] = sum_k w[n,k] * x[k] in fp64 over the fp32 dequantized row, k ascending;
 * s[n] = sum_k |w[n,k] * x[k]|. W is n_out rows of n_in/256 blocks each.
 * s may be NULL.
 */
int orc_gemv_q4k(const uint8_t *w, const float *x, int64_t n_in, int64_t n_out,
                 double *y, double *s);
int orc_gemv_iq3(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                 int64_t n_out, double *y, double *s);
int orc_gemv_iq3_xxs(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                     int64_t n_out, double *y, double *s);
int orc_gemv_iq3s(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                  int64_t n_out, double *y, double *s);
int orc_gemv_iq4xs(const uint8_t *w, const float *table, const float *x, int64_t n_in,
                   int64_t n_out, double *y, double *s);

/* Y[b, n] = sum_k w[n,k] * X[b,k], X [batch, n_in], Y and S [batch, n_out]. */
int orc_gemm_q4k(const uint8_t *w, const float *x, int64_t n_in, int64_t n_out,
                 int batch, double *y, double *s);

/* Same as the GEMVs, evaluated only for the listed rows (y, s have nrows). */
int orc_gemv_q4k_rows(const uint8_t *w, const float *x, int64_t n_in, const int64_t *rows,
                      int64_t nrows, double *y, double *s);
int orc_gemv_iq3_rows(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                      const int64_t *rows, int64_t nrows, double *y, double *s);
int orc_gemv_iq3_xxs_rows(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                          const int64_t *rows, int64_t nrows, double *y, double *s);
int orc_gemv_iq3s_rows(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                       const int64_t *rows, int64_t nrows, double *y, double *s);
int orc_gemv_iq4xs_rows(const uint8_t *w, const float *table, const float *x, int64_t n_in,
                        const int64_t *rows, int64_t nrows, double *y, double *s);

/*
 * The iq3_pack.py page's encode(): x [n_rows][n_in] fp32 (finite, n_in % 256
 * == 0) -> n_rows rows of n_in/256 98-byte blocks, with `grid` [256][4] in
 * weight units. Float32 throughout, in the order the function's comment
 * states.
 */
int orc_encode_iq3(const float *x, const float *grid, int64_t n_rows, int64_t n_in, uint8_t *dst);

/* OpenMP thread count used by the GEMVs (rows are independent, so the result
 * does not depend on it). */
void orc_set_threads(int n);
int orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
