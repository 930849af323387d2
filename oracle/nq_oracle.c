/*
 * nq_oracle.c -- the oracle for packed block-quantized weight decoding.
 * TEST INFRASTRUCTURE ONLY (see nq_oracle.h).  Shares no code, header,
 * table or generator with the HIP library.
 *
 * Each decoder below restates one rule of the ONNX page "DequantizePacked
 * decoding specification", section "Mathematical decoding rules", in that
 * section's notation: M, A, D are one binary32 multiply, add and subtract;
 * bit, field, U and P are the page's exact integer helpers; field offsets
 * come from the page's "Packed layouts and decoding" table (fields
 * concatenated in order from byte 0).  The nvfp4-with-divisor decoder
 * restates section 3.3 of the NInfer "tensor-formats" page.
 *
 * Build: gcc -O1 -std=c11 -ffp-contract=off -fno-fast-math (x86-64 SSE
 * arithmetic, so every float operation is a single IEEE binary32 operation).
 */
#include "nq_oracle.h"
#include "codebooks_hex.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Format table: DequantizePacked page, "Quantization formats" (B and S per  */
/* identifier); "nvfp4" is the NInfer section 3.3 format carried in the     */
/* gguf:nvfp4 block bytes with a 4-byte binary32 divisor after the blocks.  */
/* ------------------------------------------------------------------------ */
enum {
    F_Q4_0, F_Q4_1, F_Q5_0, F_Q5_1, F_Q8_0, F_Q8_1,
    F_Q2_K, F_Q3_K, F_Q4_K, F_Q5_K, F_Q6_K, F_Q8_K,
    F_IQ2_XXS, F_IQ2_XS, F_IQ3_XXS, F_IQ1_S, F_IQ4_NL, F_IQ3_S, F_IQ2_S, F_IQ4_XS, F_IQ1_M,
    F_TQ1_0, F_TQ2_0, F_MXFP4, F_NVFP4_GGUF, F_Q1_0, F_Q2_0,
    F_NVFP4_DIV,
    F_COUNT
};

static const struct {
    const char *name;
    int B, S, trailer;
} FORMATS[F_COUNT] = {
    {"gguf:q4_0", 32, 18, 0},     {"gguf:q4_1", 32, 20, 0},     {"gguf:q5_0", 32, 22, 0},
    {"gguf:q5_1", 32, 24, 0},     {"gguf:q8_0", 32, 34, 0},     {"gguf:q8_1", 32, 36, 0},
    {"gguf:q2_k", 256, 84, 0},    {"gguf:q3_k", 256, 110, 0},   {"gguf:q4_k", 256, 144, 0},
    {"gguf:q5_k", 256, 176, 0},   {"gguf:q6_k", 256, 210, 0},   {"gguf:q8_k", 256, 292, 0},
    {"gguf:iq2_xxs", 256, 66, 0}, {"gguf:iq2_xs", 256, 74, 0},  {"gguf:iq3_xxs", 256, 98, 0},
    {"gguf:iq1_s", 256, 50, 0},   {"gguf:iq4_nl", 32, 18, 0},   {"gguf:iq3_s", 256, 110, 0},
    {"gguf:iq2_s", 256, 82, 0},   {"gguf:iq4_xs", 256, 136, 0}, {"gguf:iq1_m", 256, 56, 0},
    {"gguf:tq1_0", 256, 54, 0},   {"gguf:tq2_0", 256, 66, 0},   {"gguf:mxfp4", 32, 17, 0},
    {"gguf:nvfp4", 64, 36, 0},    {"gguf:q1_0", 128, 18, 0},    {"gguf:q2_0", 64, 18, 0},
    {"nvfp4", 64, 36, 4},
};

int nqo_format_count(void) { return F_COUNT; }

int nqo_format_info(int fmt, const char **name, int *B, int *S, int *trailer)
{
    if (fmt < 0 || fmt >= F_COUNT) return NQO_ERR_FORMAT;
    if (name) *name = FORMATS[fmt].name;
    if (B) *B = FORMATS[fmt].B;
    if (S) *S = FORMATS[fmt].S;
    if (trailer) *trailer = FORMATS[fmt].trailer;
    return NQO_OK;
}

int nqo_format_find(const char *name)
{
    if (!name) return -1;
    for (int f = 0; f < F_COUNT; f++)
        if (strcmp(FORMATS[f].name, name) == 0) return f;
    return -1;
}

/* ------------------------------------------------------------------------ */
/* Length rule: DequantizePacked page, "Format identifiers": rank >= 1,     */
/* nonnegative dims, shape[-1] % B == 0, len = prod(shape[:-1]) *           */
/* (shape[-1]/B) * S.  Counts are exact integers; one that exceeds          */
/* INT64_MAX (the ONNX dimension type's range) is an overflow.              */
/* ------------------------------------------------------------------------ */
static int mul_ok(uint64_t a, uint64_t b, uint64_t *r)
{
    if (a != 0 && b > (uint64_t)INT64_MAX / a) return 0;
    *r = a * b;
    return 1;
}

int nqo_sizes(int fmt, const int64_t *shape, int rank, uint64_t *nbytes, uint64_t *nelems)
{
    if (fmt < 0 || fmt >= F_COUNT) return NQO_ERR_FORMAT;
    if (rank < 1 || !shape) return NQO_ERR_RANK;
    int any_zero = 0;
    for (int i = 0; i < rank; i++) {
        if (shape[i] < 0) return NQO_ERR_DIM;
        if (shape[i] == 0) any_zero = 1;
    }
    const uint64_t B = (uint64_t)FORMATS[fmt].B, S = (uint64_t)FORMATS[fmt].S;
    const uint64_t K = (uint64_t)shape[rank - 1];
    if (K % B != 0) return NQO_ERR_ALIGN;
    uint64_t elems = 0, bytes = 0;
    if (!any_zero) {
        uint64_t rows = 1; /* the product of no dimensions is 1 */
        for (int i = 0; i < rank - 1; i++)
            if (!mul_ok(rows, (uint64_t)shape[i], &rows)) return NQO_ERR_OVERFLOW;
        uint64_t blocks;
        if (!mul_ok(rows, K / B, &blocks)) return NQO_ERR_OVERFLOW;
        if (!mul_ok(blocks, S, &bytes)) return NQO_ERR_OVERFLOW;
        if (!mul_ok(rows, K, &elems)) return NQO_ERR_OVERFLOW;
        uint64_t out_bytes;
        if (!mul_ok(elems, 8, &out_bytes)) return NQO_ERR_OVERFLOW;
    }
    bytes += (uint64_t)FORMATS[fmt].trailer;
    if (bytes > (uint64_t)INT64_MAX) return NQO_ERR_OVERFLOW;
    if (nbytes) *nbytes = bytes;
    if (nelems) *nelems = elems;
    return NQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Word conversions.                                                        */
/* ------------------------------------------------------------------------ */

/* IEEE 754 binary16 -> binary32, exact: sign, 5-bit exponent (bias 15),    */
/* 10-bit fraction; exponent 0 holds zero and subnormals f * 2^-24.         */
float nqo_f16_to_f32(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    float mag;
    if (e == 0)
        mag = ldexpf((float)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexpf((float)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* binary32 -> bfloat16 with round-to-nearest, ties-to-even.  A bf16 word is */
/* the high half of a binary32 word (NInfer tensor-formats 3.1), so the two */
/* candidates are the truncated high half and its successor; the successor  */
/* of the largest finite word of a sign is that sign's infinity.  NaN stays */
/* NaN (quiet, sign kept; the page leaves the payload unspecified).         */
uint16_t nqo_f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040);
    uint32_t hi = u >> 16;
    const uint32_t lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;
    return (uint16_t)hi;
}

/* binary32 -> binary16 with round-to-nearest, ties-to-even, gradual        */
/* underflow and overflow to infinity.  Works on |x| in binary64 (exact):   */
/* scale |x| by the binary16 spacing of its binade (never below the         */
/* subnormal spacing 2^-24), round that integer ratio ties-to-even, then    */
/* encode.                                                                  */
uint16_t nqo_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
    const double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);       /* a = m * 2^e2 with m in [0.5, 1) */
    int be = e2 - 1;     /* a lies in [2^be, 2^(be+1)) */
    if (be < -14) be = -14;
    const double spacing = ldexp(1.0, be - 10);
    double n = nearbyint(a / spacing); /* default rounding: nearest, ties to even */
    if (n >= 2048.0) {   /* rounded up into the next binade */
        n = 1024.0;
        be += 1;
    }
    if (be > 15) return (uint16_t)(sign | 0x7C00u);
    if (n < 1024.0) return (uint16_t)(sign | (uint16_t)n); /* subnormal */
    return (uint16_t)(sign | (uint16_t)(((be + 15) << 10) | ((int)n - 1024)));
}

/* E4M3FN word (NInfer tensor-formats 3.3): sign bit 7, exponent bits 6:3,  */
/* fraction bits 2:0, bias 7; exponent 0 is m * 2^-9; e=15, m=7 is NaN.     */
float nqo_e4m3fn_to_f32(uint8_t w)
{
    const int sign = w >> 7, e = (w >> 3) & 15, m = w & 7;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -9);
    else if (e == 15 && m == 7)
        mag = NAN;
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -mag : mag;
}

/* bfloat16 word -> binary32 from its value classes (NInfer tensor-formats  */
/* 3.1): sign bit 15, 8-bit exponent (bias 127), 7-bit fraction; exponent 0  */
/* holds zeros and subnormals f * 2^-133, exponent 255 infinities and NaNs.  */
float nqo_bf16_to_f32(uint16_t w)
{
    const int sign = w >> 15, e = (w >> 7) & 255, f = w & 127;
    float mag;
    if (e == 0)
        mag = ldexpf((float)f, -133);
    else if (e == 255)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexpf(1.0f + (float)f / 128.0f, e - 127);
    return sign ? -mag : mag;
}

void nqo_convert(const float *x, uint64_t n, int dtype, void *out)
{
    for (uint64_t i = 0; i < n; i++) {
        switch (dtype) {
        case NQO_F32: ((float *)out)[i] = x[i]; break;
        case NQO_F16: ((uint16_t *)out)[i] = nqo_f32_to_f16(x[i]); break;
        case NQO_BF16: ((uint16_t *)out)[i] = nqo_f32_to_bf16(x[i]); break;
        case NQO_F64: ((double *)out)[i] = (double)x[i]; break;
        default: break;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* IQ codebooks: "IQ codebooks" section.  The hex bytes are split into      */
/* successive `bits`-wide fields, least significant field first in each     */
/* byte; each field indexes the signed value list; rows hold `width` values.*/
/* ------------------------------------------------------------------------ */
#define BOOK_MAX (2048 * 8)
static int8_t GRID[6][BOOK_MAX];
static int GRID_ROWS[6];
static int GRID_BAD_FIELDS;
static int grids_ready;

static int hexval(char c)
{
    if (c >= '0' && c <= '9') return c - '0';
    if (c >= 'a' && c <= 'f') return c - 'a' + 10;
    return -1;
}

static void expand_grids(void)
{
    if (grids_ready) return;
    GRID_BAD_FIELDS = 0;
    for (int k = 0; k < 6; k++) {
        const nqo_codebook_text *t = &NQO_CODEBOOK_TEXT[k];
        const size_t nbytes = strlen(t->hex) / 2;
        const size_t nfields = nbytes * 8 / (size_t)t->bits;
        for (size_t f = 0; f < nfields && f < BOOK_MAX; f++) {
            const size_t bitpos = f * (size_t)t->bits;
            const int byte = hexval(t->hex[2 * (bitpos / 8)]) * 16 + hexval(t->hex[2 * (bitpos / 8) + 1]);
            const int field = (byte >> (bitpos % 8)) & ((1 << t->bits) - 1);
            if (field >= t->nvalues) {
                GRID_BAD_FIELDS++;
                GRID[k][f] = 0;
            } else {
                GRID[k][f] = (int8_t)t->values[field];
            }
        }
        GRID_ROWS[k] = (int)(nfields / (size_t)t->width);
    }
    grids_ready = 1;
}

int nqo_grid_rows(int book)
{
    expand_grids();
    return (book >= 0 && book < 6) ? GRID_ROWS[book] : 0;
}

int nqo_grid_width(int book) { return (book >= 0 && book < 6) ? NQO_CODEBOOK_TEXT[book].width : 0; }

int nqo_grid_value(int book, int row, int j)
{
    expand_grids();
    if (book < 0 || book >= 6 || row < 0 || row >= GRID_ROWS[book] || j < 0 ||
        j >= NQO_CODEBOOK_TEXT[book].width)
        return -1000;
    return GRID[book][row * NQO_CODEBOOK_TEXT[book].width + j];
}

int nqo_grid_bad_fields(void)
{
    expand_grids();
    return GRID_BAD_FIELDS;
}

enum { IQ2XXS, IQ2XS, IQ2S, IQ3XXS, IQ3S, IQ1S };

/* G(name, r): row r of a codebook. */
static const int8_t *G(int book, int r) { return &GRID[book][r * NQO_CODEBOOK_TEXT[book].width]; }

/* ------------------------------------------------------------------------ */
/* The page's notation: "Mathematical decoding rules".                      */
/* ------------------------------------------------------------------------ */
static float M(float a, float b) { return a * b; }
static float A(float a, float b) { return a + b; }
static float D(float a, float b) { return a - b; }

/* bit(v,k) = floor(v / 2^k) mod 2;  field(v,k,w) = floor(v / 2^k) mod 2^w */
static unsigned bit(uint64_t v, int k) { return (unsigned)((v >> k) & 1u); }
static unsigned field(uint64_t v, int k, int w) { return (unsigned)((v >> k) & ((1ull << w) - 1u)); }

/* U(a): unsigned little-endian integer of a byte sequence. */
static uint64_t U(const uint8_t *a, int n)
{
    uint64_t v = 0;
    for (int i = 0; i < n; i++) v |= (uint64_t)a[i] << (8 * i);
    return v;
}

/* Floating-point fields are converted exactly to FLOAT before use. */
static float H(const uint8_t *a) { return nqo_f16_to_f32((uint16_t)U(a, 2)); }
static float R32(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* P(a,w,g): byte-group starts s = 0, g, 2g, ...; bit planes p = 0..8/w-1; */
/* byte positions j = 0..g-1; element field(a[s+j], w*p, w).               */
static int P(const uint8_t *a, int len, int w, int g, int *out)
{
    int n = 0;
    for (int s = 0; s < len; s += g)
        for (int p = 0; p < 8 / w; p++)
            for (int j = 0; j < g; j++) out[n++] = (int)field(a[s + j], w * p, w);
    return n;
}

static int signed8(uint8_t v) { return v >= 128 ? (int)v - 256 : (int)v; }

/* IQ4_NL table and the doubled E2M1 table V (both zero entries are +0). */
static const int IQ4[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
static const int V[16] = {0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12};

/* --- Conventional and nonlinear formats --------------------------------- */
/* Q4_0: h d; u8 q[16]        Q4_1: h d,m; u8 q[16]                         */
/* Q5_0: h d; u8 high[4],q[16]  Q5_1: h d,m; u8 high[4],q[16]   IQ4_NL: as Q4_0 */
static void dec_conventional(int fmt, const uint8_t *b, float *y)
{
    const float d = H(b);
    float m = 0.0f;
    const uint8_t *q;
    uint64_t high = 0;
    int v[32];
    switch (fmt) {
    case F_Q4_0: case F_IQ4_NL: q = b + 2; break;
    case F_Q4_1: m = H(b + 2); q = b + 4; break;
    case F_Q5_0: high = U(b + 2, 4); q = b + 6; break;
    default: /* F_Q5_1 */ m = H(b + 2); high = U(b + 4, 4); q = b + 8; break;
    }
    P(q, 16, 4, 16, v);
    if (fmt == F_Q5_0 || fmt == F_Q5_1)
        for (int j = 0; j < 32; j++) v[j] = v[j] + 16 * (int)bit(high, j);
    for (int j = 0; j < 32; j++) {
        switch (fmt) {
        case F_Q4_0: y[j] = M(d, (float)(v[j] - 8)); break;
        case F_Q4_1: y[j] = A(M(d, (float)v[j]), m); break;
        case F_Q5_0: y[j] = M(d, (float)(v[j] - 16)); break;
        case F_Q5_1: y[j] = A(M(d, (float)v[j]), m); break;
        default: /* IQ4_NL */ y[j] = M(d, (float)IQ4[v[j]]); break;
        }
    }
}

/* Q8_0: h d; i8 q[32]   Q8_1: h d,s; i8 q[32]   Q8_K: f d; i8 q[256]; i16 sums[16] */
/* y[j] = M(d, q[j]); the cached s and sums never enter.                    */
static void dec_q8(int fmt, const uint8_t *b, float *y)
{
    float d;
    const uint8_t *q;
    int n;
    if (fmt == F_Q8_0) { d = H(b); q = b + 2; n = 32; }
    else if (fmt == F_Q8_1) { d = H(b); q = b + 4; n = 32; }
    else { d = R32((uint32_t)U(b, 4)); q = b + 4; n = 256; }
    for (int j = 0; j < n; j++) y[j] = M(d, (float)signed8(q[j]));
}

/* Q1_0: h d; u8 q[16]: y[j] = d if bit(q[floor(j/8)], j mod 8) else -d.  */
static void dec_q1_0(const uint8_t *b, float *y)
{
    const float d = H(b);
    for (int j = 0; j < 128; j++) y[j] = bit(b[2 + j / 8], j % 8) ? d : -d;
}

/* Q2_0: h d; u8 q[16]: v = P(q,2,1), y[j] = M(d, v[j] - 1). */
static void dec_q2_0(const uint8_t *b, float *y)
{
    const float d = H(b);
    int v[64];
    P(b + 2, 16, 2, 1, v);
    for (int j = 0; j < 64; j++) y[j] = M(d, (float)(v[j] - 1));
}

/* --- K-quant formats and IQ4_XS ----------------------------------------- */
/* Q2_K: u8 scales[16],q[64]; h d,dmin                                       */
static void dec_q2_k(const uint8_t *b, float *y)
{
    const uint8_t *scales = b, *q = b + 16;
    const float d = H(b + 80), dmin = H(b + 82);
    int v[256];
    P(q, 64, 2, 32, v);
    for (int j = 0; j < 256; j++) {
        const int s = scales[j / 16];
        y[j] = D(M(M(d, (float)(s % 16)), (float)v[j]), M(dmin, (float)(s / 16)));
    }
}

/* Q3_K: u8 mask[32],q[64],scales[12]; h d                                   */
static void dec_q3_k(const uint8_t *b, float *y)
{
    const uint8_t *mask = b, *q = b + 32;
    const float d = H(b + 108);
    int v[256], h[256], l[16], a[16];
    P(q, 64, 2, 32, v);
    P(mask, 32, 1, 32, h);
    P(b + 96, 8, 4, 8, l);
    P(b + 104, 4, 2, 4, a);
    for (int j = 0; j < 256; j++) {
        const int k = j / 16;
        const int s = l[k] + 16 * a[k] - 32;
        y[j] = M(M(d, (float)s), (float)(v[j] - 4 * (1 - h[j])));
    }
}

/* Q4_K: h d,dmin; u8 scales[12],q[128]                                      */
/* Q5_K: h d,dmin; u8 scales[12],high[32],q[128]                             */
static void dec_q45_k(int fmt, const uint8_t *b, float *y)
{
    const float d = H(b), dmin = H(b + 2);
    const uint8_t *s = b + 4;
    const uint8_t *q = (fmt == F_Q4_K) ? b + 16 : b + 48;
    int v[256], a[8], m[8];
    P(q, 128, 4, 32, v);
    if (fmt == F_Q5_K) {
        int hb[256];
        P(b + 16, 32, 1, 32, hb);
        for (int j = 0; j < 256; j++) v[j] = v[j] + 16 * hb[j];
    }
    for (int k = 0; k < 8; k++) {
        if (k < 4) {
            a[k] = s[k] % 64;
            m[k] = s[k + 4] % 64;
        } else {
            a[k] = (s[k + 4] % 16) + 16 * (s[k - 4] / 64);
            m[k] = (s[k + 4] / 16) + 16 * (s[k] / 64);
        }
    }
    for (int j = 0; j < 256; j++) {
        const int k = j / 32;
        y[j] = D(M(M(d, (float)a[k]), (float)v[j]), M(dmin, (float)m[k]));
    }
}

/* Q6_K: u8 low[128],high[64]; i8 scales[16]; h d                            */
static void dec_q6_k(const uint8_t *b, float *y)
{
    const uint8_t *low = b, *high = b + 128, *scales = b + 192;
    const float d = H(b + 208);
    int l[256], h[256];
    P(low, 128, 4, 64, l);
    P(high, 64, 2, 32, h);
    for (int j = 0; j < 256; j++) {
        const int s = signed8(scales[j / 16]);
        y[j] = M(M(d, (float)s), (float)(l[j] + 16 * h[j] - 32));
    }
}

/* IQ4_XS: h d; u16 high; u8 scales[4],q[128].  The garbled scale formula   */
/* reads s[k] = field(scales[k/2], 4(k mod 2), 4) + 16 field(high, 2k, 2) - 32. */
static void dec_iq4_xs(const uint8_t *b, float *y)
{
    const float d = H(b);
    const uint64_t high = U(b + 2, 2);
    const uint8_t *scales = b + 4, *q = b + 8;
    int v[256], s[8];
    P(q, 128, 4, 16, v);
    for (int k = 0; k < 8; k++)
        s[k] = (int)field(scales[k / 2], 4 * (k % 2), 4) + 16 * (int)field(high, 2 * k, 2) - 32;
    for (int j = 0; j < 256; j++) y[j] = M(M(d, (float)s[j / 32]), (float)IQ4[v[j]]);
}

/* --- IQ2, IQ3 and IQ1 formats ------------------------------------------- */
/* S(v): signs 1 - 2 bit(v,j); SP(v): seven stored bits plus their parity.  */
static void S_signs(unsigned v, int *s)
{
    for (int j = 0; j < 8; j++) s[j] = 1 - 2 * (int)bit(v, j);
}

static void SP_signs(unsigned v, int *s)
{
    unsigned parity = 0;
    for (int j = 0; j < 7; j++) {
        s[j] = 1 - 2 * (int)bit(v, j);
        parity += bit(v, j);
    }
    s[7] = 1 - 2 * (int)(parity % 2);
}

static void dec_iq23(int fmt, const uint8_t *b, float *y)
{
    const float d = H(b);
    for (int g = 0; g < 8; g++) {
        for (int l = 0; l < 4; l++) {
            const int i = 4 * g + l;
            int v[8], s[8];
            float c;
            switch (fmt) {
            case F_IQ2_XXS: {
                const uint64_t a = U(b + 6 + 8 * g, 4);
                const int8_t *row = G(IQ2XXS, b[2 + 8 * g + l]);
                for (int j = 0; j < 8; j++) v[j] = row[j];
                SP_signs(field(a, 7 * l, 7), s);
                c = M(M(d, 0.5f + (float)(a >> 28)), 0.25f);
                break;
            }
            case F_IQ2_XS: {
                const uint64_t a = U(b + 2 + 2 * i, 2);
                const unsigned t = field(b[66 + g], 4 * (l / 2), 4);
                const int8_t *row = G(IQ2XS, (int)(a % 512));
                for (int j = 0; j < 8; j++) v[j] = row[j];
                SP_signs((unsigned)(a / 512), s);
                c = M(M(d, 0.5f + (float)t), 0.25f);
                break;
            }
            case F_IQ2_S: {
                const int r = b[2 + i] + 256 * (int)field(b[66 + g], 2 * l, 2);
                const unsigned t = field(b[74 + g], 4 * (l / 2), 4);
                const int8_t *row = G(IQ2S, r);
                for (int j = 0; j < 8; j++) v[j] = row[j];
                S_signs(b[34 + i], s);
                c = M(M(d, 0.5f + (float)t), 0.25f);
                break;
            }
            case F_IQ3_XXS: {
                const uint64_t a = U(b + 66 + 4 * g, 4);
                const int8_t *r0 = G(IQ3XXS, b[2 + 2 * i]), *r1 = G(IQ3XXS, b[3 + 2 * i]);
                for (int j = 0; j < 4; j++) { v[j] = r0[j]; v[4 + j] = r1[j]; }
                SP_signs(field(a, 7 * l, 7), s);
                c = M(M(d, 0.5f + (float)(a >> 28)), 0.5f);
                break;
            }
            default: { /* F_IQ3_S */
                int r[2];
                for (int t = 0; t < 2; t++) r[t] = b[2 + 2 * i + t] + 256 * (int)bit(b[66 + g], 2 * l + t);
                const int8_t *r0 = G(IQ3S, r[0]), *r1 = G(IQ3S, r[1]);
                for (int j = 0; j < 4; j++) { v[j] = r0[j]; v[4 + j] = r1[j]; }
                S_signs(b[74 + i], s);
                c = M(d, (float)(1 + 2 * (int)field(b[106 + g / 2], 4 * (g % 2), 4)));
                break;
            }
            }
            for (int j = 0; j < 8; j++) y[8 * i + j] = M(M(c, (float)v[j]), (float)s[j]);
        }
    }
}

/* IQ1_S: h d; u8 q[32]; u16 high[8]      IQ1_M: u8 q[32],high[16],scales[8] */
static void dec_iq1(int fmt, const uint8_t *b, float *y)
{
    float d = 0.0f;
    uint64_t w[4] = {0, 0, 0, 0};
    if (fmt == F_IQ1_S) {
        d = H(b);
    } else {
        for (int k = 0; k < 4; k++) w[k] = U(b + 48 + 2 * k, 2);
        uint64_t bits = 0;
        for (int k = 0; k < 4; k++) bits += (w[k] >> 12) << (4 * k);
        d = nqo_f16_to_f32((uint16_t)bits);
    }
    for (int g = 0; g < 8; g++) {
        for (int l = 0; l < 4; l++) {
            const int i = 4 * g + l;
            int r;
            float c, delta;
            if (fmt == F_IQ1_S) {
                const uint64_t a = U(b + 34 + 2 * g, 2);
                r = b[2 + i] + 256 * (int)field(a, 3 * l, 3);
                c = M(d, (float)(2 * (int)field(a, 12, 3) + 1));
                delta = bit(a, 15) ? -0.125f : 0.125f;
            } else {
                const unsigned a = field(b[32 + i / 2], 4 * (i % 2), 4);
                r = b[i] + 256 * (int)(a % 8);
                const unsigned t = field(w[g / 2], 6 * (g % 2) + 3 * (l / 2), 3);
                c = M(d, (float)(2 * (int)t + 1));
                delta = bit(a, 3) ? -0.125f : 0.125f;
            }
            const int8_t *v = G(IQ1S, r);
            for (int j = 0; j < 8; j++) y[8 * i + j] = M(c, A((float)v[j], delta));
        }
    }
}

/* --- Ternary and block-floating formats --------------------------------- */
/* TQ1_0: u8 q[48],high[4]; h d.  Sequences (start,width,count) = (0,32,5), */
/* (32,16,5), (48,4,4); p before j; t = floor(3((b*3^p) mod 256)/256) - 1.  */
static void dec_tq1_0(const uint8_t *b, float *y)
{
    static const int SEQ[3][3] = {{0, 32, 5}, {32, 16, 5}, {48, 4, 4}};
    const float d = H(b + 52);
    int n = 0;
    for (int k = 0; k < 3; k++) {
        const int start = SEQ[k][0], width = SEQ[k][1], count = SEQ[k][2];
        for (int p = 0; p < count; p++) {
            int pow3 = 1;
            for (int e = 0; e < p; e++) pow3 *= 3;
            for (int j = 0; j < width; j++) {
                const int t = (3 * ((b[start + j] * pow3) % 256)) / 256 - 1;
                y[n++] = M(d, (float)t);
            }
        }
    }
}

/* TQ2_0: u8 q[64]; h d: y[j] = M(d, v[j] - 1), v = P(q,2,32). */
static void dec_tq2_0(const uint8_t *b, float *y)
{
    const float d = H(b + 64);
    int v[256];
    P(b, 64, 2, 32, v);
    for (int j = 0; j < 256; j++) y[j] = M(d, (float)(v[j] - 1));
}

/* MXFP4: u8 exponent,q[16].  Half scale d has bit pattern 0x00200000 * 2^e */
/* for e < 2 and (e-1) * 2^23 otherwise; y[j] = M(d, V[v[j]]), v = P(q,4,16). */
static void dec_mxfp4(const uint8_t *b, float *y)
{
    const unsigned e = b[0];
    const float d = R32(e < 2 ? 0x00200000u << e : (e - 1u) << 23);
    int v[32];
    P(b + 1, 16, 4, 16, v);
    for (int j = 0; j < 32; j++) y[j] = M(d, (float)V[v[j]]);
}

/* NVFP4 (gguf): u8 scales[4],q[32]; four groups of 16.  Half scale: zero   */
/* for the whole byte 0 or 127, m * 2^-10 for E = 0, (1 + m/8) 2^(E-8) else, */
/* with E = field(e,3,4), m = e mod 8 (bit 7 enters neither).               */
static float nvfp4_half_scale(unsigned e)
{
    const unsigned E = field(e, 3, 4), m = e % 8;
    if (e == 0 || e == 127) return 0.0f;
    if (E == 0) return ldexpf((float)m, -10);
    return ldexpf(1.0f + (float)m / 8.0f, (int)E - 8);
}

static void dec_nvfp4_gguf(const uint8_t *b, float *y)
{
    for (int g = 0; g < 4; g++) {
        const float d = nvfp4_half_scale(b[g]);
        int v[16];
        P(b + 4 + 8 * g, 8, 4, 8, v);
        for (int j = 0; j < 16; j++) y[16 * g + j] = M(d, (float)V[v[j]]);
    }
}

/* nvfp4 with divisor (NInfer tensor-formats 3.3): W = e2m1(c) * e4m3fn(s) / d_w. */
/* E2M1: sign bit 3, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (code 8 is -0).   */
/* Codes and scale words sit where gguf:nvfp4 puts them.                    */
static float e2m1(unsigned c)
{
    static const float MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const float mag = MAG[c & 7];
    return (c & 8) ? -mag : mag;
}

static void dec_nvfp4_div(const uint8_t *b, float d_w, float *y)
{
    for (int g = 0; g < 4; g++) {
        const float s = nqo_e4m3fn_to_f32(b[g]);
        int v[16];
        P(b + 4 + 8 * g, 8, 4, 8, v);
        for (int j = 0; j < 16; j++) {
            const float p = M(e2m1((unsigned)v[j]), s); /* exact: <= 6 significant bits */
            y[16 * g + j] = p / d_w;                     /* one correctly rounded division */
        }
    }
}

static void decode_block(int fmt, const uint8_t *b, float d_w, float *y)
{
    switch (fmt) {
    case F_Q4_0: case F_Q4_1: case F_Q5_0: case F_Q5_1: case F_IQ4_NL: dec_conventional(fmt, b, y); break;
    case F_Q8_0: case F_Q8_1: case F_Q8_K: dec_q8(fmt, b, y); break;
    case F_Q1_0: dec_q1_0(b, y); break;
    case F_Q2_0: dec_q2_0(b, y); break;
    case F_Q2_K: dec_q2_k(b, y); break;
    case F_Q3_K: dec_q3_k(b, y); break;
    case F_Q4_K: case F_Q5_K: dec_q45_k(fmt, b, y); break;
    case F_Q6_K: dec_q6_k(b, y); break;
    case F_IQ4_XS: dec_iq4_xs(b, y); break;
    case F_IQ2_XXS: case F_IQ2_XS: case F_IQ2_S: case F_IQ3_XXS: case F_IQ3_S: dec_iq23(fmt, b, y); break;
    case F_IQ1_S: case F_IQ1_M: dec_iq1(fmt, b, y); break;
    case F_TQ1_0: dec_tq1_0(b, y); break;
    case F_TQ2_0: dec_tq2_0(b, y); break;
    case F_MXFP4: dec_mxfp4(b, y); break;
    case F_NVFP4_GGUF: dec_nvfp4_gguf(b, y); break;
    case F_NVFP4_DIV: dec_nvfp4_div(b, d_w, y); break;
    default: break;
    }
}

int nqo_decode_blocks_f32(int fmt, const uint8_t *blocks, uint64_t nblocks, float d_w, float *y)
{
    if (fmt < 0 || fmt >= F_COUNT) return NQO_ERR_FORMAT;
    expand_grids();
    const uint64_t B = (uint64_t)FORMATS[fmt].B, S = (uint64_t)FORMATS[fmt].S;
    for (uint64_t i = 0; i < nblocks; i++) decode_block(fmt, blocks + i * S, d_w, y + i * B);
    return NQO_OK;
}

/* Signature and storage: blocks decode in input order to FLOAT, the values */
/* are reshaped to `shape` (row-major, a no-op on the flat order) and       */
/* converted once to the output type.                                       */
int nqo_decode(int fmt, const uint8_t *payload, uint64_t nbytes, const int64_t *shape, int rank,
               int dtype, void *out)
{
    if (dtype < NQO_F32 || dtype > NQO_F64) return NQO_ERR_DTYPE;
    uint64_t need = 0, nelems = 0;
    const int st = nqo_sizes(fmt, shape, rank, &need, &nelems);
    if (st != NQO_OK) return st;
    if (need != nbytes) return NQO_ERR_LENGTH;
    expand_grids();
    const uint64_t B = (uint64_t)FORMATS[fmt].B, S = (uint64_t)FORMATS[fmt].S;
    const uint64_t nblocks = nelems / B;
    float d_w = 0.0f;
    if (FORMATS[fmt].trailer == 4) d_w = R32((uint32_t)U(payload + nbytes - 4, 4));
    static const int OSIZE[4] = {4, 2, 2, 8};
    float y[256];
    for (uint64_t i = 0; i < nblocks; i++) {
        decode_block(fmt, payload + i * S, d_w, y);
        nqo_convert(y, B, dtype, (uint8_t *)out + i * B * (uint64_t)OSIZE[dtype]);
    }
    return NQO_OK;
}

/* Stacked nvfp4 (NInfer tensor-formats 3.3).  The rows of the plane are the  */
/* N = prod(shape[:-1]) rows of the flat row-major layout; row n takes the   */
/* divisor of its source, d_w[floor(n / (N / divisors))], and each of its    */
/* blocks is decoded with that divisor.                                      */
int nqo_sizes_nvfp4_stacked(const int64_t *shape, int rank, int64_t divisors, uint64_t *nbytes,
                            uint64_t *nelems)
{
    uint64_t nb1 = 0, ne = 0;
    const int st = nqo_sizes(F_NVFP4_DIV, shape, rank, &nb1, &ne);
    if (st != NQO_OK) return st;
    if (divisors < 1) return NQO_ERR_DIVISORS;
    uint64_t rows = 1; /* N = prod(shape[:-1]), the product of no dimensions being 1 */
    for (int i = 0; i + 1 < rank; i++)
        if (!mul_ok(rows, (uint64_t)shape[i], &rows)) return NQO_ERR_OVERFLOW;
    if (rows % (uint64_t)divisors != 0) return NQO_ERR_DIVISORS;
    if ((uint64_t)divisors > (0x7FFFFFFFFFFFFFFFull - (nb1 - 4)) / 4) return NQO_ERR_OVERFLOW;
    if (nbytes) *nbytes = nb1 - 4 + 4 * (uint64_t)divisors;
    if (nelems) *nelems = ne;
    return NQO_OK;
}

int nqo_decode_nvfp4_stacked(const uint8_t *payload, uint64_t nbytes, const int64_t *shape, int rank,
                             int64_t divisors, int dtype, void *out)
{
    if (dtype < NQO_F32 || dtype > NQO_F64) return NQO_ERR_DTYPE;
    uint64_t need = 0, nelems = 0;
    const int st = nqo_sizes_nvfp4_stacked(shape, rank, divisors, &need, &nelems);
    if (st != NQO_OK) return st;
    if (need != nbytes) return NQO_ERR_LENGTH;
    if (nelems == 0) return NQO_OK;
    const uint64_t K = (uint64_t)shape[rank - 1];
    const uint64_t N = nelems / K;
    const uint64_t rows_per_source = N / (uint64_t)divisors;
    const uint64_t blocks_per_row = K / 64;
    const uint8_t *trailer = payload + N * blocks_per_row * 36;
    static const int OSIZE[4] = {4, 2, 2, 8};
    float y[64];
    for (uint64_t n = 0; n < N; n++) {
        const float d_w = R32((uint32_t)U(trailer + 4 * (n / rows_per_source), 4));
        for (uint64_t b = 0; b < blocks_per_row; b++) {
            const uint64_t i = n * blocks_per_row + b;
            dec_nvfp4_div(payload + i * 36, d_w, y);
            nqo_convert(y, 64, dtype, (uint8_t *)out + i * 64 * (uint64_t)OSIZE[dtype]);
        }
    }
    return NQO_OK;
}

/* Row-scaled FP8 (NInfer tensor-formats 3.3): w_hat[n,k] = binary32(c32 *   */
/* s32) with c32 the exact E4M3FN value of code c[n,k] and s32 the exact     */
/* binary32 value of row n's bfloat16 (kind 0) or binary16 (kind 1) scale.   */
int nqo_sizes_fp8_row(const int64_t *shape, int rank, uint64_t *nbytes, uint64_t *nelems)
{
    if (rank != 2 || !shape) return NQO_ERR_RANK;
    if (shape[0] <= 0 || shape[1] <= 0) return NQO_ERR_DIM; /* positive dimensions */
    uint64_t elems, out_bytes, scale_bytes, bytes;
    if (!mul_ok((uint64_t)shape[0], (uint64_t)shape[1], &elems)) return NQO_ERR_OVERFLOW;
    if (!mul_ok(elems, 8, &out_bytes)) return NQO_ERR_OVERFLOW;
    if (!mul_ok((uint64_t)shape[0], 2, &scale_bytes)) return NQO_ERR_OVERFLOW;
    bytes = elems + scale_bytes;
    if (bytes < elems || bytes > (uint64_t)INT64_MAX) return NQO_ERR_OVERFLOW;
    if (nbytes) *nbytes = bytes;
    if (nelems) *nelems = elems;
    return NQO_OK;
}

int nqo_decode_fp8_row(int scale_kind, const uint8_t *payload, uint64_t nbytes, const int64_t *shape,
                       int rank, int dtype, void *out)
{
    if (scale_kind != 0 && scale_kind != 1) return NQO_ERR_FORMAT;
    if (dtype < NQO_F32 || dtype > NQO_F64) return NQO_ERR_DTYPE;
    uint64_t need = 0, nelems = 0;
    const int st = nqo_sizes_fp8_row(shape, rank, &need, &nelems);
    if (st != NQO_OK) return st;
    if (need != nbytes) return NQO_ERR_LENGTH;
    const uint64_t N = (uint64_t)shape[0], K = (uint64_t)shape[1];
    const uint8_t *scales = payload + N * K;
    static const int OSIZE[4] = {4, 2, 2, 8};
    for (uint64_t n = 0; n < N; n++) {
        const uint16_t sw = (uint16_t)U(scales + 2 * n, 2);
        const float s32 = scale_kind == 0 ? nqo_bf16_to_f32(sw) : nqo_f16_to_f32(sw);
        for (uint64_t k = 0; k < K; k++) {
            const float w = M(nqo_e4m3fn_to_f32(payload[n * K + k]), s32);
            nqo_convert(&w, 1, dtype, (uint8_t *)out + (n * K + k) * (uint64_t)OSIZE[dtype]);
        }
    }
    return NQO_OK;
}

/* grouped_absmax (NInfer tensor-formats 7.2), step by step for one group of */
/* binary32 values: amax of |x|; an all-zero group gives scale +0 and codes  */
/* 0; otherwise raw = RN32(amax / qmax), scale16 = RN16(raw) with 0x0001 in   */
/* place of +0 and failure on a non-finite scale, inv = RN32(1 / scale32),    */
/* and each code is RN-to-integral-ties-even(RN32(x * inv)) clamped to        */
/* [qmin, qmax].  The divisor is qmax, not |qmin|.                            */
static const struct { int G, qmin, qmax; } GQ_SCHEMES[4] = {
    {64, -8, 7}, {64, -16, 15}, {64, -32, 31}, {32, -127, 127}};

static float gq_source(int in_dtype, const void *x, uint64_t i)
{
    switch (in_dtype) {
    case 0: return ((const float *)x)[i];
    case 1: return nqo_f16_to_f32(((const uint16_t *)x)[i]);
    case 2: return nqo_bf16_to_f32(((const uint16_t *)x)[i]);
    default: return (float)((const double *)x)[i]; /* C conversion: round to nearest even */
    }
}

static int gq_group(int scheme, const float *v, int n, int8_t *code, uint16_t *scale)
{
    const int qmin = GQ_SCHEMES[scheme].qmin, qmax = GQ_SCHEMES[scheme].qmax;
    int status = 0;
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        if (!isfinite(v[i])) status |= 1;
        const float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (status) return status;
    if (amax == 0.0f) {
        *scale = 0x0000;
        for (int i = 0; i < n; i++) code[i] = 0;
        return 0;
    }
    const float raw = amax / (float)qmax;
    uint16_t s16 = nqo_f32_to_f16(raw);
    if (s16 == 0x0000) s16 = 0x0001; /* 2^-24 underflow rescue */
    if ((s16 & 0x7C00) == 0x7C00) return 2;
    *scale = s16;
    const float inv = 1.0f / nqo_f16_to_f32(s16);
    for (int i = 0; i < n; i++) {
        const float r = rintf(v[i] * inv); /* default rounding: nearest, ties to even */
        code[i] = (int8_t)(r < (float)qmin ? qmin : r > (float)qmax ? qmax : (int)r);
    }
    return 0;
}

int nqo_grouped_absmax(int scheme, int in_dtype, const void *x, int64_t N, int64_t K, int8_t *codes,
                       uint16_t *scales)
{
    if (scheme < 0 || scheme > 3 || in_dtype < 0 || in_dtype > 3 || N <= 0 || K <= 0) return -1;
    const int G = GQ_SCHEMES[scheme].G;
    const int64_t ng = (K + G - 1) / G;
    float v[64];
    int status = 0;
    for (int64_t n = 0; n < N; n++)
        for (int64_t g = 0; g < ng; g++) {
            const int64_t k0 = g * G;
            const int cnt = (int)(K - k0 < G ? K - k0 : G);
            for (int i = 0; i < cnt; i++) v[i] = gq_source(in_dtype, x, (uint64_t)(n * K + k0 + i));
            status |= gq_group(scheme, v, cnt, codes + n * K + k0, scales + n * ng + g);
        }
    return status;
}

/* ------------------------------------------------------------------------- */
/* Linear products with q8_1 activations (NInfer tensor-formats: the         */
/* paragraph on products over gguf_* weights -- the activation becomes ggml  */
/* q8_1 numbers, one binary16 scale and one sum per 32 values, and products  */
/* accumulate in FP32 -- and the consumer paragraph of the conformance       */
/* section: reduction order and intermediate precision are the kernel's, and */
/* the Op result is judged against an independent oracle under a named       */
/* criterion).                                                               */
/*                                                                           */
/* Activation quantizer.  The pages name the q8_1 numbers but not the rule   */
/* that assigns them; this oracle uses the 8-bit, 32-value absmax rule of    */
/* section 7.2 (q8_g32_fp16, gq_group above) for the codes and the scale d,  */
/* and stores as the sum field RN16(d32 * (sum of the 32 codes)): the        */
/* binary16 of the block's represented sum.  d32 has at most 11 significant  */
/* bits and |sum| <= 32 * 127 < 2^12, so that product is exact in binary32   */
/* and the field takes one rounding.  Blocks are gguf q8_1 blocks (packed-   */
/* layout table of the DequantizePacked page): d at byte 0, the sum at 2,    */
/* the 32 signed codes at 4..35.                                             */
int nqo_quantize_q8_1(int in_dtype, const void *x, int64_t M, int64_t K, uint8_t *blocks)
{
    if (in_dtype < 0 || in_dtype > 3 || M <= 0 || K <= 0 || K % 32 != 0) return -1;
    const int64_t kb = K / 32;
    int status = 0;
    float v[32];
    int8_t q[32];
    for (int64_t m = 0; m < M; m++)
        for (int64_t c = 0; c < kb; c++) {
            uint8_t *b = blocks + (uint64_t)(m * kb + c) * 36u;
            for (int i = 0; i < 32; i++) v[i] = gq_source(in_dtype, x, (uint64_t)(m * K + c * 32 + i));
            uint16_t d16 = 0;
            const int st = gq_group(3, v, 32, q, &d16);
            if (st) { /* the encoder fails: the block is unspecified (zeroed here) */
                status |= st;
                memset(b, 0, 36);
                continue;
            }
            int sum = 0;
            for (int i = 0; i < 32; i++) sum += q[i];
            const uint16_t s16 = nqo_f32_to_f16(nqo_f16_to_f32(d16) * (float)sum);
            if ((s16 & 0x7C00) == 0x7C00) status |= 4;
            b[0] = (uint8_t)(d16 & 0xFF);
            b[1] = (uint8_t)(d16 >> 8);
            b[2] = (uint8_t)(s16 & 0xFF);
            b[3] = (uint8_t)(s16 >> 8);
            for (int i = 0; i < 32; i++) b[4 + i] = (uint8_t)q[i];
        }
    return status;
}

/* Code bytes of the formats whose decode formula adds a term that does not  */
/* depend on the weight's own code (q4_1 and q5_1: + m; q2_k, q4_k, q5_k:   */
/* - RN32(dmin * m_sub)), from the packed-layout table.  With those bytes    */
/* zeroed every code is 0 and the block decodes to exactly that term.        */
static int offset_code_bytes(int fmt, int *lo, int *hi)
{
    switch (fmt) {
    case F_Q4_1: *lo = 4; *hi = 20; return 1;   /* q@4..19 */
    case F_Q5_1: *lo = 4; *hi = 24; return 1;   /* high@4..7, q@8..23 */
    case F_Q2_K: *lo = 16; *hi = 80; return 1;  /* q@16..79 */
    case F_Q4_K: *lo = 16; *hi = 144; return 1; /* q@16..143 */
    case F_Q5_K: *lo = 16; *hi = 176; return 1; /* high@16..47, q@48..175 */
    default: return 0;
    }
}

/* The product y[m][n] = sum_k w[n][k] * x[m][k] of a gguf_* weight [N, K]   */
/* (each value the format's decoded binary32 weight) and M q8_1 activation   */
/* rows of K values (each d32 * q, exact in binary32), in binary64: every    */
/* product is exact (at most 24 + 18 significant bits) and the sum runs in k */
/* order.  env[m][n] = sum_k |x[m][k]| * E[n][k], the scale of the error     */
/* criterion, with E = |w| for formats whose value is a scale times a code   */
/* and E = |w| + 2 |o| for the five formats above (o: the code-independent   */
/* term), since a kernel may sum the scaled codes and that term apart and    */
/* |scale * code| + |o| <= |w| + 2 |o|.                                      */
int nqo_gemv_q8_1(int fmt, const uint8_t *w, uint64_t nbytes, int64_t N, int64_t K, const uint8_t *xq,
                  int64_t M, double *y, double *env)
{
    if (fmt < 0 || fmt >= (int)(sizeof FORMATS / sizeof FORMATS[0]) || FORMATS[fmt].trailer != 0)
        return NQO_ERR_FORMAT;
    if (N <= 0 || K <= 0 || M <= 0) return NQO_ERR_DIM;
    if (K % 32 != 0) return NQO_ERR_ALIGN;
    const int64_t wshape[2] = {N, K}, xshape[2] = {M, K};
    uint64_t need = 0, ne = 0, xbytes = 0;
    int st = nqo_sizes(fmt, wshape, 2, &need, &ne);
    if (st != NQO_OK) return st;
    if (need != nbytes) return NQO_ERR_LENGTH;
    st = nqo_sizes(F_Q8_1, xshape, 2, &xbytes, NULL);
    if (st != NQO_OK) return st;
    float *wh = malloc((size_t)(N * K) * sizeof(float));
    float *o = calloc((size_t)(N * K), sizeof(float));
    float *xh = malloc((size_t)(M * K) * sizeof(float));
    uint8_t *wz = NULL;
    if (!wh || !o || !xh) { st = NQO_ERR_OVERFLOW; goto done; }
    if ((st = nqo_decode(fmt, w, nbytes, wshape, 2, NQO_F32, wh)) != NQO_OK) goto done;
    if ((st = nqo_decode(F_Q8_1, xq, xbytes, xshape, 2, NQO_F32, xh)) != NQO_OK) goto done;
    int lo, hi;
    if (offset_code_bytes(fmt, &lo, &hi)) {
        const uint64_t S = (uint64_t)FORMATS[fmt].S;
        if (!(wz = malloc(nbytes))) { st = NQO_ERR_OVERFLOW; goto done; }
        memcpy(wz, w, nbytes);
        for (uint64_t b = 0; b < nbytes / S; b++) memset(wz + b * S + lo, 0, (size_t)(hi - lo));
        if ((st = nqo_decode(fmt, wz, nbytes, wshape, 2, NQO_F32, o)) != NQO_OK) goto done;
    }
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, e = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const double wv = wh[n * K + k], xv = xh[m * K + k];
                acc += wv * xv;
                e += fabs(xv) * (fabs(wv) + 2.0 * fabs((double)o[n * K + k]));
            }
            y[m * N + n] = acc;
            if (env) env[m * N + n] = e;
        }
done:
    free(wh);
    free(o);
    free(xh);
    free(wz);
    return st;
}
