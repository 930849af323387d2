/*
 * nq.h -- C ABI of the MI355X (gfx950) packed-weight decoder.
 *
 * The operation is DequantizePacked as defined by the ONNX page
 * "DequantizePacked decoding specification" (opset 29), section "Signature and
 * storage": a rank-one payload of packed bytes, a format identifier and a
 * logical shape decode, block by block in input order, to binary32 values
 * that are reshaped to `shape` (row-major) and converted once to the output
 * type, with round-to-nearest-even for FLOAT16 and BFLOAT16.  The formats
 * are the 27 "gguf:" profiles of that page's identifier table and "nvfp4",
 * the FP32-divisor format of section 3.3 of the NInfer "tensor-formats" page
 * (stored as gguf:nvfp4 blocks followed by one little-endian binary32
 * divisor; see nq_dequantize_packed).
 *
 * Every entry point is reentrant and keeps no mutable global state beyond a
 * per-device cache of the compute-unit count.  No entry point allocates,
 * frees or retains caller memory.
 */
#ifndef NQ_H
#define NQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every metadata error is detected on the host before any
 * launch, so a call failing with any status but NQ_ERR_HIP has written
 * nothing (NQ_ERR_HIP: see nq_dequantize_packed). */
typedef enum {
    NQ_OK = 0,
    NQ_ERR_NULL_ARG = 1,          /* a required pointer is NULL */
    NQ_ERR_UNKNOWN_FORMAT = 2,    /* name or id outside the closed registry */
    NQ_ERR_BAD_RANK = 3,          /* rank < 1 */
    NQ_ERR_BAD_DIM = 4,           /* a negative dimension (or a count outside its range) */
    NQ_ERR_NOT_BLOCK_ALIGNED = 5, /* shape[rank-1] % B != 0 (also for empty tensors) */
    NQ_ERR_LENGTH_MISMATCH = 6,   /* nbytes differs from the length rule */
    NQ_ERR_OVERFLOW = 7,          /* byte count, or element count * 8, beyond INT64_MAX */
    NQ_ERR_BAD_DTYPE = 8,         /* out_dtype not one of nq_dtype */
    NQ_ERR_HIP = 9,               /* the HIP runtime reported an error at launch */
    NQ_ERR_BAD_DIVISORS = 10,     /* stacked nvfp4: divisors < 1, above 2^30, or not dividing the rows */
    NQ_ERR_MISALIGNED = 11,       /* a pointer lacks the alignment the call requires */
    NQ_ERR_SCRATCH = 12           /* nq_gemm_q8_1_noalloc: the shape needs more than NQ_GEMM_SCRATCH_BYTES */
} nq_status;

/* Output types: the page's FLOAT, FLOAT16, BFLOAT16 and DOUBLE. */
typedef enum { NQ_F32 = 0, NQ_F16 = 1, NQ_BF16 = 2, NQ_F64 = 3 } nq_dtype;

/* Kernel family a format decodes in. */
typedef enum {
    NQ_FAMILY_SIMPLE = 0,  /* 32/64/128-value blocks: q4_0..q8_1, iq4_nl, q1_0, q2_0 */
    NQ_FAMILY_KQUANT = 1,  /* 256-value super-blocks: q2_k..q8_k, iq4_xs */
    NQ_FAMILY_IQ = 2,      /* codebook formats: iq2_xxs, iq2_xs, iq2_s, iq3_xxs, iq3_s, iq1_s, iq1_m */
    NQ_FAMILY_FP4 = 3,     /* gguf:mxfp4, gguf:nvfp4, nvfp4 */
    NQ_FAMILY_TERNARY = 4  /* tq1_0, tq2_0 */
} nq_family;

typedef struct {
    int32_t id;            /* 0 .. nq_format_count()-1 */
    const char *name;      /* static string, e.g. "gguf:q4_k" */
    int32_t block_values;  /* B */
    int32_t block_bytes;   /* S */
    int32_t trailer_bytes; /* bytes after the last block: 4 for "nvfp4", else 0 */
    int32_t family;        /* nq_family */
} nq_format_info;

/* Number of registered formats (28): the 27 identifiers of the
 * DequantizePacked page's "Format identifiers" table and "nvfp4". */
int nq_format_count(void);

/* Registry entry by id: ids 0..26 follow the order of the DequantizePacked
 * page's "Format identifiers" table, id 27 is "nvfp4"; B and S are the
 * page's "Quantization formats" block values and bytes.  NQ_ERR_NULL_ARG if
 * out is NULL, NQ_ERR_UNKNOWN_FORMAT if id is out of range. */
int nq_format_by_id(int32_t id, nq_format_info *out);

/* Registry entry by identifier: exact, case-sensitive match of one of the
 * page's identifiers ("gguf:q4_0" ... "gguf:q2_0") or "nvfp4".  Other
 * spellings, including parameterized ones, are NQ_ERR_UNKNOWN_FORMAT
 * (DequantizePacked page, "Format identifiers"). */
int nq_format_query(const char *name, nq_format_info *out);

/* Host-only metadata check (no device access).  Applies the length rule of
 * the DequantizePacked page, "Format identifiers": rank >= 1, every dimension
 * >= 0, shape[rank-1] % B == 0 (also when another dimension is zero), and
 * nbytes == prod(shape[:-1]) * (shape[-1] / B) * S, plus 4 trailer bytes for
 * "nvfp4" (present even for an empty tensor).  On success stores the element
 * count and the output byte count for out_dtype (either pointer may be
 * NULL).  shape may be NULL only when rank < 1 (then NQ_ERR_BAD_RANK). */
int nq_validate(int32_t format, uint64_t nbytes, const int64_t *shape, int32_t rank,
                int32_t out_dtype, uint64_t *out_elems, uint64_t *out_bytes);

/* Decode a payload into `out`, asynchronously on `stream`.
 *
 *   format    registry id (nq_format_query)
 *   payload   device pointer to nbytes packed bytes, any alignment; block i
 *             occupies bytes [i*S, (i+1)*S).  For "nvfp4" the last 4 bytes are
 *             the binary32 divisor d_w.  May be NULL only if nbytes == 0.
 *   shape     host array of `rank` int64 dimensions (ONNX order, last
 *             dimension contiguous)
 *   out_dtype nq_dtype
 *   out       device pointer to prod(shape) elements of out_dtype, aligned to
 *             the element size (else NQ_ERR_MISALIGNED); 16-byte alignment
 *             takes the vector-store path.  May be NULL only if prod(shape)
 *             == 0.  Must not overlap payload.
 *   stream    HIP stream (0 for the null stream)
 *
 * Element j of block i is out[i*B + j]: y = DequantizePacked(x) in the flat
 * row-major order of `shape`.  Ownership stays with the caller; nothing is
 * retained after return.  The call validates as nq_validate, returns NQ_OK
 * without launching for an empty tensor, and otherwise enqueues the decode
 * and returns NQ_OK, or NQ_ERR_HIP if the launch failed.  A tensor of more
 * than 2^30 units (8 values) or 2^32 payload bytes is decoded by several
 * launches on `stream`; NQ_ERR_HIP from a later one leaves the earlier ones'
 * outputs enqueued (written once the stream reaches them).  Payload bytes are
 * never inspected on the host: every byte pattern of the "gguf:" formats
 * decodes; for "nvfp4" only sign-zero finite E4M3FN scales and a finite
 * positive divisor are valid words (NInfer page, section 3.3), and other
 * words decode deterministically by the same formula. */
int nq_dequantize_packed(int32_t format, const void *payload, uint64_t nbytes, const int64_t *shape,
                         int32_t rank, int32_t out_dtype, void *out, hipStream_t stream);

/* One tensor of a many-tensor decode. */
typedef struct {
    int32_t format;         /* registry id */
    int32_t rank;           /* >= 1 */
    const int64_t *shape;   /* host array of `rank` dimensions */
    const void *payload;    /* device, nbytes packed bytes, any alignment */
    uint64_t nbytes;
    void *out;              /* device, prod(shape) elements of the call's out_dtype */
} nq_tensor;

/* Decode `count` tensors to out_dtype on `stream`: the same output, bit for
 * bit, as nq_dequantize_packed on each tensor in turn (DequantizePacked
 * page, "Signature and storage"; a model's weight set is many such
 * tensors), in fewer launches: the tensors of one format (and one output
 * alignment class) share launches of up to 64 tensors each, so that small
 * tensors fill the device together instead of one launch at a time.
 *
 * Every tensor is validated first, as nq_validate with out_dtype plus the
 * pointer rules of nq_dequantize_packed (NULL payload with nbytes > 0 or
 * NULL out with elements: NQ_ERR_NULL_ARG; out not element-aligned:
 * NQ_ERR_MISALIGNED); on the first failure the call returns its status,
 * stores its index in *failed (when failed is not NULL; -1 otherwise and on
 * success) and launches nothing.  count < 0 is NQ_ERR_BAD_DIM, tensors NULL
 * with count > 0 NQ_ERR_NULL_ARG, a bad out_dtype NQ_ERR_BAD_DTYPE; count ==
 * 0 and empty tensors launch nothing.  No output may overlap another output
 * or any payload.  NQ_ERR_HIP reports a failed launch; the launches before
 * it stay enqueued.  The caller owns every buffer and the tensor array,
 * which is not retained after return; nothing is allocated on the device. */
int nq_dequantize_packed_many(const nq_tensor *tensors, int32_t count, int32_t out_dtype, int32_t *failed,
                              hipStream_t stream);

/* "nvfp4" planes stacked from several source matrices (NInfer
 * "tensor-formats" page, section 3.3): such a plane carries one binary32
 * weight divisor per source.  With N = prod(shape[:-1]) rows, source j covers
 * the N / divisors consecutive rows from row j * (N / divisors) on, and
 * every value of row n is e2m1(c) * e4m3fn(s) / d_w[floor(n / (N / divisors))]
 * (one correctly rounded binary32 division).
 *
 * Layout (the page leaves the placement of the divisors open): the
 * gguf:nvfp4 blocks of all rows, then `divisors` little-endian binary32
 * words in stacking order; divisors == 1 is exactly the "nvfp4" format.
 * Length rule: nbytes == N * (shape[-1] / 64) * 36 + 4 * divisors.
 *
 * nq_validate_nvfp4_stacked checks, in this order: out_dtype, rank >= 1,
 * shape != NULL, dimensions >= 0, shape[-1] % 64 == 0, 1 <= divisors <= 2^30
 * (NQ_ERR_BAD_DIVISORS), the counts (NQ_ERR_OVERFLOW as nq_validate), N %
 * divisors == 0 (NQ_ERR_BAD_DIVISORS; N may be 0), then nbytes; on success it
 * stores the element and output byte counts (either pointer may be NULL).
 * nq_dequantize_nvfp4_stacked validates the same way, then behaves as
 * nq_dequantize_packed for "nvfp4": asynchronous on `stream`, nothing
 * launched for an empty tensor, the same pointer and alignment rules, the
 * same ownership (the caller's buffers are neither retained nor freed). */
int nq_validate_nvfp4_stacked(uint64_t nbytes, const int64_t *shape, int32_t rank, int64_t divisors,
                              int32_t out_dtype, uint64_t *out_elems, uint64_t *out_bytes);
int nq_dequantize_nvfp4_stacked(const void *payload, uint64_t nbytes, const int64_t *shape, int32_t rank,
                                int64_t divisors, int32_t out_dtype, void *out, hipStream_t stream);

/* Row-scaled FP8 (NInfer "tensor-formats" page, section 3.3):
 * fp8_e4m3fn_row_bf16 (scale_kind NQ_FP8_ROW_BF16) and fp8_e4m3fn_row_fp16
 * (NQ_FP8_ROW_FP16).  A rank-two [N, K] matrix, both dimensions positive;
 * value [n, k] is the binary32 product of E4M3FN code c[n, k] and row n's
 * bfloat16 / binary16 multiplier, converted once to out_dtype (RNE for
 * f16/bf16, exact for f64).
 *
 * Layout (the page defers it to a layout registry it does not print): the
 * N*K code bytes row-major, then N little-endian 16-bit scale words in row
 * order.  Length rule: nbytes == N*K + 2*N.
 *
 * nq_validate_fp8_row checks, in this order: scale_kind
 * (NQ_ERR_UNKNOWN_FORMAT), out_dtype, rank == 2 (NQ_ERR_BAD_RANK), shape !=
 * NULL, both dimensions > 0 (NQ_ERR_BAD_DIM), N*K*8 and nbytes within
 * INT64_MAX (NQ_ERR_OVERFLOW), then nbytes.  nq_dequantize_fp8_row validates
 * the same way and then follows nq_dequantize_packed: asynchronous on
 * `stream`, payload of any alignment (NULL refused), `out` element-aligned
 * (NQ_ERR_MISALIGNED otherwise; 16-byte alignment takes the vector stores), caller-owned buffers neither
 * retained nor freed.  Code words 0x7F/0xFF (NaN) and refused scale words
 * (negative, non-finite) decode by the same formula. */
typedef enum { NQ_FP8_ROW_BF16 = 0, NQ_FP8_ROW_FP16 = 1 } nq_fp8_row_scale;

int nq_validate_fp8_row(int32_t scale_kind, uint64_t nbytes, const int64_t *shape, int32_t rank,
                        int32_t out_dtype, uint64_t *out_elems, uint64_t *out_bytes);
int nq_dequantize_fp8_row(int32_t scale_kind, const void *payload, uint64_t nbytes, const int64_t *shape,
                          int32_t rank, int32_t out_dtype, void *out, hipStream_t stream);

/* grouped_absmax encoder (NInfer "tensor-formats" page, section 7.2) for the
 * grouped integer schemes: q4_g64_fp16 (codes -8..7, 64 columns per group),
 * q5_g64_fp16 (-16..15), q6_g64_fp16 (-32..31), q8_g32_fp16 (-127..127, 32
 * per group).  For each row and group of a [N, K] source matrix: amax of
 * |x|; an all-zero group gives scale +0 and zero codes; otherwise raw =
 * RN32(amax / qmax), scale16 = RN16(raw) (0x0001 if that is +0), inv =
 * RN32(1 / scale32) and code = clamp(round-half-even(RN32(x * inv)), qmin,
 * qmax).  Sources of in_dtype f16/bf16/f64 are converted to binary32 first
 * (RNE).
 *
 * Outputs (the page leaves the packed row-split layout undefined): `codes`,
 * N*K signed bytes row-major; `scales`, N*ceil(K/G) binary16 words row-major
 * (the last group of a row may be short).  `status` is one device uint32:
 * the call first clears it on `stream`, then ORs in 1 if a source value is
 * not finite in binary32 and 2 if a scale rounds past binary16 (the encoder
 * "fails"; the codes and scales of such groups are then unspecified).  Read
 * it after the stream reaches this point.
 *
 * nq_validate_grouped_absmax checks, in this order: scheme
 * (NQ_ERR_UNKNOWN_FORMAT), in_dtype (NQ_ERR_BAD_DTYPE), rank == 2
 * (NQ_ERR_BAD_RANK), shape != NULL, both dimensions > 0 (NQ_ERR_BAD_DIM),
 * K < 2^31 and the byte counts within INT64_MAX (NQ_ERR_OVERFLOW); it stores
 * the byte sizes of codes and scales (either pointer may be NULL).
 * nq_quantize_grouped_absmax validates the same way, then requires x,
 * codes, scales and status non-NULL (NQ_ERR_NULL_ARG), x aligned to its
 * element size, scales to 2 bytes and status to 4 (NQ_ERR_MISALIGNED), and
 * enqueues the encoder;
 * the caller owns every buffer.  x must not overlap the outputs. */
typedef enum { NQ_GQ_Q4_G64 = 0, NQ_GQ_Q5_G64 = 1, NQ_GQ_Q6_G64 = 2, NQ_GQ_Q8_G32 = 3 } nq_grouped_scheme;

int nq_validate_grouped_absmax(int32_t scheme, const int64_t *shape, int32_t rank, int32_t in_dtype,
                               uint64_t *codes_bytes, uint64_t *scales_bytes);
int nq_quantize_grouped_absmax(int32_t scheme, const void *x, const int64_t *shape, int32_t rank, int32_t in_dtype,
                               void *codes, void *scales, uint32_t *status, hipStream_t stream);

/* Products with q8_1 activations (NInfer "tensor-formats" page: a product
 * over a gguf_* weight quantizes the activation to ggml q8_1 numbers, one
 * binary16 scale and one sum per 32 values, and accumulates in FP32; the
 * kernel's reduction order and intermediate precision are its own, and the
 * result is judged against an independent oracle under a named criterion).
 *
 * nq_quantize_q8_1: a [M, K] activation (shape[0] = M rows, shape[1] = K,
 * K % 32 == 0; in_dtype f32/f16/bf16/f64, converted to binary32 with RNE)
 * becomes M*K/32 gguf q8_1 blocks of 36 bytes, row-major (block c of row m at
 * byte 36*(m*K/32 + c)): binary16 d at byte 0, binary16 sum at 2, 32 signed
 * codes at 4.  The pages name q8_1 numbers but not the rule that assigns
 * them; the codes and d follow the q8_g32_fp16 rule of section 7.2 (see
 * nq_quantize_grouped_absmax), and the sum is RN16(d32 * sum of the codes),
 * a product exact in binary32.  `status` (one device uint32) is cleared on
 * `stream` first, then ORed with 1 for a non-finite source, 2 for a scale
 * past binary16 (that block is then all zero bytes) and 4 for a sum past
 * binary16 (the sum field is then infinite).
 * nq_validate_quantize_q8_1 checks in_dtype (NQ_ERR_BAD_DTYPE), rank == 2
 * (NQ_ERR_BAD_RANK), shape (NQ_ERR_NULL_ARG), both dimensions > 0
 * (NQ_ERR_BAD_DIM), K % 32 (NQ_ERR_NOT_BLOCK_ALIGNED) and the byte counts
 * (NQ_ERR_OVERFLOW), and stores the blocks' byte size.  nq_quantize_q8_1
 * also requires x, blocks and status non-NULL (NQ_ERR_NULL_ARG), x aligned
 * to its element size and blocks and status to 4 bytes (NQ_ERR_MISALIGNED).
 * The caller owns every
 * buffer; x must not overlap the outputs.
 *
 * nq_gemv_q8_1: y[m*N + n] = sum_k w[n][k] * x[m][k] (binary32 output,
 * row-major [M, N]) for a gguf_* weight payload of N rows of K values
 * (`format` one of the 27 "gguf:" ids, nbytes = N * (K/B) * S) and M q8_1
 * activation rows as nq_quantize_q8_1 writes them, 1 <= M <= 8; w is the
 * format's decoded binary32 weight and x[m][k] = d32 * code.  Accumulation
 * is binary32 with fused multiply-adds in an order fixed per launch shape, so
 * repeated calls give identical bits; against the exact sum the error stays
 * below gamma(K + 8) * sum_k |x| E + (K + 8) * 2^-148, gamma(n) = n u /
 * (1 - n u), u = 2^-24, with E = |w|, or |w| + 2|o| for q4_1, q5_1, q2_k,
 * q4_k and q5_k (o: the weight's value at code 0).
 * nq_validate_gemv_q8_1 checks the format (NQ_ERR_UNKNOWN_FORMAT, also for
 * "nvfp4"), N, K > 0 and 1 <= M <= 8 (NQ_ERR_BAD_DIM), K % B
 * (NQ_ERR_NOT_BLOCK_ALIGNED), N, K < 2^31 (NQ_ERR_OVERFLOW) and nbytes
 * (NQ_ERR_LENGTH_MISMATCH).  nq_gemv_q8_1 also requires weight, xq and y
 * non-NULL (NQ_ERR_NULL_ARG) and xq and y aligned to 4 bytes
 * (NQ_ERR_MISALIGNED), then enqueues
 * the product on `stream`.  The caller owns every buffer; y must not overlap
 * the inputs. */
int nq_validate_quantize_q8_1(const int64_t *shape, int32_t rank, int32_t in_dtype, uint64_t *blocks_bytes);
int nq_quantize_q8_1(const void *x, const int64_t *shape, int32_t rank, int32_t in_dtype, void *blocks,
                     uint32_t *status, hipStream_t stream);
int nq_validate_gemv_q8_1(int32_t format, uint64_t nbytes, int64_t N, int64_t K, int64_t M);
int nq_gemv_q8_1(int32_t format, const void *weight, uint64_t nbytes, int64_t N, int64_t K, const void *xq,
                 int64_t M, float *y, hipStream_t stream);

/* nq_gemm_q8_1: the same product for any number of activation rows M >= 1
 * (the page's GGUF linear operation over a batch), with the same argument
 * meaning, layouts and criterion.  Up to 4 rows it makes the launch
 * nq_gemv_q8_1 makes (identical bits); with 5 or more rows every 32 weight
 * values become signed 8-bit codes with a binary32 scale (and an offset for
 * q4_1, q5_1, q2_k, q4_k and q5_k), their exact integer dot products with
 * the activation codes come from the 8-bit matrix cores, and each is scaled
 * and added in binary32 (tiles of 16, 32 or 64 activation rows by M; K in
 * steps of 256 values, or 128 on grids of more than two 64-row tiles per
 * compute unit and with K split over five eighths to two of them).
 * When the output has few tiles and K is long, K is split over workgroups:
 * each split's partial output goes to `workspace` (device memory the caller
 * owns, at least the size nq_gemm_q8_1_workspace reports, 16-byte aligned,
 * not overlapping the other buffers, and not used by another call until
 * this call's work on `stream` is done), and the partials are summed in
 * split order by a second launch.  Above 256 activation rows (384 for
 * gguf:q4_k, gguf:q2_k, gguf:tq2_0 and gguf:q8_k) the weight's 8-bit codes,
 * scales and offsets are also written there once per call (same values, same
 * bits).  With workspace NULL or smaller than that size
 * the product runs unsplit and without the once-per-call rewrite.  Repeated
 * calls with the same shape, device and workspace choice (given or not)
 * give identical bits.
 * nq_validate_gemm_q8_1 checks as nq_validate_gemv_q8_1 except that M may
 * be any count >= 1 below 2^31 with M * K / 32 * 36 and M * N * 4 below 2^63
 * (NQ_ERR_OVERFLOW).  nq_gemm_q8_1_workspace runs the same checks (nbytes
 * taken as the format's length rule) and stores the workspace size for the
 * shape on the current device (0 when the product would neither split K nor
 * rewrite the weight once; `bytes` NULL: NQ_ERR_NULL_ARG).  nq_gemm_q8_1
 * requires weight, xq and y non-NULL (NQ_ERR_NULL_ARG) and xq and y aligned
 * to 4 bytes and workspace to 16 (NQ_ERR_MISALIGNED), then
 * enqueues the product on `stream`.  The caller owns every buffer; y must not
 * overlap the inputs. */
int nq_validate_gemm_q8_1(int32_t format, uint64_t nbytes, int64_t N, int64_t K, int64_t M);
int nq_gemm_q8_1_workspace(int32_t format, int64_t N, int64_t K, int64_t M, uint64_t *bytes);
int nq_gemm_q8_1(int32_t format, const void *weight, uint64_t nbytes, int64_t N, int64_t K, const void *xq,
                 int64_t M, float *y, void *workspace, uint64_t workspace_bytes, hipStream_t stream);

/* nq_gemm_q8_1_noalloc: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The same product, argument meaning, checks and result as
 * nq_gemm_q8_1 called with a workspace of the size nq_gemm_q8_1_workspace
 * reports (the same bits), but the workspace is the library's own static
 * device scratch of NQ_GEMM_SCRATCH_BYTES: every GPU the library is loaded
 * on holds one from load until the process ends.  The call allocates
 * nothing.  A shape whose workspace exceeds the scratch is refused with
 * NQ_ERR_SCRATCH before anything is launched (at that size: every
 * Llama-3-8B-shaped weight with up to 256 activation rows fits; larger
 * batches, whose weight is rewritten once per call, need nq_gemm_q8_1 and a
 * workspace); NQ_ERR_HIP if the scratch's device address cannot be found.
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents (nothing in it has to start at zero): calls ordered on one stream
 * are safe, calls that may overlap on one GPU (other streams, other host
 * threads) race and their outputs are undefined. */
#define NQ_GEMM_SCRATCH_BYTES (32u << 20)
int nq_gemm_q8_1_noalloc(int32_t format, const void *weight, uint64_t nbytes, int64_t N, int64_t K, const void *xq,
                         int64_t M, float *y, hipStream_t stream);

/* Static description of a status code (the nq_status values above; other
 * values give "unknown status").  The pages define no status codes: these
 * are the library's names for the failures its checks detect. */
const char *nq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
