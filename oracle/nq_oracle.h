/*
 * nq_oracle -- plain, slow, single-threaded CPU decoder for packed
 * block-quantized weights.  TEST INFRASTRUCTURE ONLY: the product library
 * never links, loads or calls it; only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark do.
 *
 * What it computes is defined by two pages:
 *   - ONNX "DequantizePacked decoding specification" (opset 29): the
 *     signature and storage rules, the format identifier table, the packed
 *     layout table, the binary32 rounding rules and the "Mathematical
 *     decoding rules" (conventional, K-quant, IQ and ternary/block-floating
 *     subsections), the IQ codebooks;
 *   - NInfer "tensor-formats" maintainer page, section 3.3 (nvfp4 with an
 *     FP32 weight divisor), 3.1 (bf16 words), 3.2 (fp32 words).
 *
 * Every floating-point operation is one IEEE binary32 operation rounded to
 * nearest-even with gradual underflow (built with -ffp-contract=off and no
 * fast-math); nothing is fused or reassociated.
 */
#ifndef NQ_ORACLE_H
#define NQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes of the oracle's own length rule. */
enum {
    NQO_OK = 0,
    NQO_ERR_FORMAT = 1,   /* index out of range */
    NQO_ERR_RANK = 2,     /* rank < 1 */
    NQO_ERR_DIM = 3,      /* a negative dimension */
    NQO_ERR_ALIGN = 4,    /* shape[-1] % B != 0 */
    NQO_ERR_OVERFLOW = 5, /* a byte or element count beyond INT64_MAX */
    NQO_ERR_LENGTH = 6,   /* nbytes differs from the length rule */
    NQO_ERR_DTYPE = 7,    /* unknown output dtype */
    NQO_ERR_DIVISORS = 8  /* divisors < 1, or the row count is not a multiple of it */
};

/* Output dtypes: 0 binary32, 1 binary16, 2 bfloat16, 3 binary64. */
enum { NQO_F32 = 0, NQO_F16 = 1, NQO_BF16 = 2, NQO_F64 = 3 };

/* Format table: index -> (name, B values per block, S bytes per block,
 * trailer bytes after the blocks).  28 entries: the 27 "gguf:" profiles of
 * the identifier table and "nvfp4" (block bytes as gguf:nvfp4 plus a
 * trailing little-endian binary32 divisor). */
int nqo_format_count(void);
int nqo_format_info(int fmt, const char **name, int *B, int *S, int *trailer);
int nqo_format_find(const char *name); /* exact, case-sensitive; -1 if absent */

/* Length rule: nbytes = prod(shape[:-1]) * (shape[-1] / B) * S (+ trailer). */
int nqo_sizes(int fmt, const int64_t *shape, int rank, uint64_t *nbytes, uint64_t *nelems);

/* Decode a whole payload.  out holds prod(shape) values of `dtype`. */
int nqo_decode(int fmt, const uint8_t *payload, uint64_t nbytes, const int64_t *shape,
               int rank, int dtype, void *out);

/* "nvfp4" with stacked divisors (NInfer tensor-formats section 3.3): a plane
 * of N = prod(shape[:-1]) rows assembled from `divisors` source matrices
 * holds one binary32 weight divisor per source; source j covers the N /
 * divisors consecutive rows starting at row j * (N / divisors), and row n
 * is divided by d_w[floor(n / (N / divisors))].  Bytes: the gguf:nvfp4
 * blocks of all rows, then the `divisors` little-endian binary32 words in
 * stacking order.  divisors == 1 is the plain "nvfp4" format. */
int nqo_sizes_nvfp4_stacked(const int64_t *shape, int rank, int64_t divisors, uint64_t *nbytes,
                            uint64_t *nelems);
int nqo_decode_nvfp4_stacked(const uint8_t *payload, uint64_t nbytes, const int64_t *shape, int rank,
                             int64_t divisors, int dtype, void *out);

/* Row-scaled FP8 (NInfer tensor-formats section 3.3): fp8_e4m3fn_row_bf16
 * (scale_kind 0) and fp8_e4m3fn_row_fp16 (scale_kind 1).  A rank-two [N, K]
 * matrix with positive dimensions; every weight is one E4M3FN code word and
 * every row one bfloat16 / binary16 multiplier; the value is the binary32
 * product code * scale.  Bytes (the page leaves the layout to an undefined
 * layout registry): the N*K codes row-major, then the N scale words,
 * little-endian 16-bit, in row order.  nbytes = N*K + 2*N. */
int nqo_sizes_fp8_row(const int64_t *shape, int rank, uint64_t *nbytes, uint64_t *nelems);
int nqo_decode_fp8_row(int scale_kind, const uint8_t *payload, uint64_t nbytes, const int64_t *shape,
                       int rank, int dtype, void *out);

/* grouped_absmax encoder (NInfer tensor-formats section 7.2) for the grouped
 * integer schemes 0 q4_g64_fp16, 1 q5_g64_fp16, 2 q6_g64_fp16, 3 q8_g32_fp16:
 * a positive [N, K] matrix of source values (in_dtype 0 binary32, 1 binary16,
 * 2 bfloat16, 3 binary64, converted to binary32 with round-to-nearest-even)
 * becomes one signed code per value (codes[n*K + k], one byte each) and one
 * binary16 scale per row and group of G columns (scales[n*ceil(K/G) + g]; the
 * last group of a row may be short).  Returns -1 for a bad scheme, dtype or
 * shape, else status bits: 1 a source value that is not finite in binary32,
 * 2 a scale that does not fit binary16 (outputs are then unspecified). */
int nqo_grouped_absmax(int scheme, int in_dtype, const void *x, int64_t N, int64_t K, int8_t *codes,
                       uint16_t *scales);

/* Linear products with q8_1 activations (NInfer "tensor-formats": products
 * over gguf_* weights quantize the activation to q8_1 numbers and accumulate
 * in FP32; the Op is judged against an independent oracle).
 *
 * nqo_quantize_q8_1: M rows of K source values (K % 32 == 0; in_dtype as in
 * nqo_grouped_absmax) become M*K/32 gguf q8_1 blocks of 36 bytes (binary16 d
 * at 0, binary16 sum at 2, 32 signed codes at 4): codes and d by the
 * q8_g32_fp16 rule of section 7.2, sum = RN16(d32 * sum of codes).  Returns
 * -1 for bad arguments, else status bits: 1 a non-finite source, 2 a scale
 * past binary16 (that block is zeroed), 4 a sum past binary16.
 *
 * nqo_gemv_q8_1: y[m*N + n] = sum_k w[n][k] * x[m][k] in binary64 for a
 * gguf_* weight [N, K] and q8_1 activations [M, K]; env[m*N + n] (may be
 * NULL) = sum_k |x| * E, E = |w| + 2|o| where o is the code-independent term
 * of q4_1, q5_1, q2_k, q4_k and q5_k, E = |w| otherwise.  Returns an
 * NQO_ERR_* code (NQO_ERR_FORMAT for "nvfp4" and out-of-range indices,
 * NQO_ERR_ALIGN for K % 32 != 0). */
int nqo_quantize_q8_1(int in_dtype, const void *x, int64_t M, int64_t K, uint8_t *blocks);
int nqo_gemv_q8_1(int fmt, const uint8_t *w, uint64_t nbytes, int64_t N, int64_t K, const uint8_t *xq,
                  int64_t M, double *y, double *env);

/* Decode `nblocks` back-to-back blocks to binary32 (no trailer; `d_w` is the
 * divisor used by "nvfp4" and ignored by every other format). */
int nqo_decode_blocks_f32(int fmt, const uint8_t *blocks, uint64_t nblocks, float d_w, float *y);

/* Scalar word conversions, each written from its IEEE / page definition. */
float nqo_f16_to_f32(uint16_t h);
uint16_t nqo_f32_to_bf16(float x);
uint16_t nqo_f32_to_f16(float x);
float nqo_e4m3fn_to_f32(uint8_t w);
float nqo_bf16_to_f32(uint16_t w);
void nqo_convert(const float *x, uint64_t n, int dtype, void *out);

/* Expanded IQ codebooks: book 0..5 = iq2xxs, iq2xs, iq2s, iq3xxs, iq3s, iq1s. */
int nqo_grid_rows(int book);
int nqo_grid_width(int book);
int nqo_grid_value(int book, int row, int j);
int nqo_grid_bad_fields(void); /* packed fields that index past the value list */

#ifdef __cplusplus
}
#endif
#endif
