// nq_gqenc.h -- grouped_absmax encoder (q4/q5/q6_g64_fp16, q8_g32_fp16).
//
// NInfer "tensor-formats" page, section 7.2: for every row and group of G
// columns of a [N, K] matrix of binary32 source values, amax = max |x|; an
// all-zero group gets scale +0 and zero codes; otherwise raw = RN32(amax /
// qmax), scale16 = RN16(raw) (0x0001 in place of +0; an infinite scale fails),
// inv = RN32(1 / scale32) and code = clamp(round-half-even(RN32(x * inv)),
// qmin, qmax).  Sources of binary16, bfloat16 or binary64 are first converted
// to binary32 with round-to-nearest-even; a source that is not finite in
// binary32 fails.
//
// Output (the page leaves the row-split layout's bytes undefined): one signed
// code byte per value, codes[n*K + k], and one binary16 scale per row and
// group, scales[n*ceil(K/G) + g]; the last group of a row may be short.
//
// Work split: a lane encodes VPL consecutive values of one group (32 source
// bytes: 8 binary32, 16 binary16/bfloat16 or 4 binary64 values); the G/VPL
// lanes of a group are consecutive lanes of a wave and reduce amax (with the
// failure test folded in) with cross-lane exchanges.  A wave's source loads and code stores are
// contiguous.  Failures set bits of a caller-owned status word with an
// atomic OR.
#pragma once

#include "nq_kernel.h"

namespace nq {

struct GqScheme {
    int G, qmin, qmax;
};
constexpr GqScheme GQ[4] = {{64, -8, 7}, {64, -16, 15}, {64, -32, 31}, {32, -127, 127}};

struct GqArgs {
    const void *x;      // source value (row r0, column 0) of this launch
    int8_t *codes;      // code of that value
    uint16_t *scales;   // scale of the launch's first group
    uint32_t *status;   // bit 0: non-finite source, bit 1: scale past binary16
    uint32_t K;         // columns (row length)
    uint32_t ngr;       // groups per row, ceil(K / G)
    uint32_t ngroups;   // groups in this launch (rows * ngr <= 2^30)
    uint32_t gmul, gshift;  // division by ngr as a multiply-shift (div_magic)
};

// Source element i (from x) as binary32: exact for binary16 and bfloat16,
// round-to-nearest-even for binary64.
template <int IN>
NQ_HD float gq_word_to_f32(const void *x, uint64_t i) {
    if constexpr (IN == 0)
        return ((const float *)x)[i];
    else if constexpr (IN == 1)
        return f16(((const uint16_t *)x)[i]);
    else if constexpr (IN == 2)
        return bits_f32((uint32_t)((const uint16_t *)x)[i] << 16);
    else
        return (float)((const double *)x)[i];
}

// Values per lane: 32 source bytes (two 16-byte loads) per lane, so that
// each load instruction of a wave covers 64 lanes at a 32-byte stride
// (measured: 16 values of a 4-byte source per lane, at a 64-byte stride, is
// 23% slower; 8 values of a 2-byte source, 16% slower than 16).
template <int IN>
constexpr int gq_vpl() {
    return IN == 0 ? 8 : IN == 3 ? 4 : 16;
}

// Source reader of the kernels: element by element, or a lane's VPL values
// with 16-byte loads when they start on a 16-byte boundary.
struct GqDevSrc {
    const void *x;
    template <int IN>
    NQ_HD float one(uint64_t i) const { return gq_word_to_f32<IN>(x, i); }
    template <int IN>
    NQ_HD void span(uint64_t i, float (&v)[gq_vpl<IN>()]) const {
        constexpr int GQ_VPL = gq_vpl<IN>();
        constexpr int ESZ = IN == 0 ? 4 : IN == 3 ? 8 : 2;
        constexpr int NV = GQ_VPL * ESZ / 16;  // 16-byte loads
        u32x4 w[NV];
        const u32x4 *p = (const u32x4 *)((const uint8_t *)x + i * ESZ);
#pragma unroll
        for (int k = 0; k < NV; k++) {
#if defined(__HIP_DEVICE_COMPILE__)
            w[k] = __builtin_nontemporal_load(p + k);
#else
            w[k] = p[k];
#endif
        }
        const uint32_t *d = (const uint32_t *)w;
#pragma unroll
        for (int k = 0; k < GQ_VPL; k++) {
            if constexpr (IN == 0)
                v[k] = bits_f32(d[k]);
            else if constexpr (IN == 1)
                v[k] = f16((d[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
            else if constexpr (IN == 2)
                v[k] = bits_f32((d[k >> 1] >> (16 * (k & 1))) << 16);
            else
                v[k] = (float)__builtin_bit_cast(double, (uint64_t)d[2 * k] | ((uint64_t)d[2 * k + 1] << 32));
        }
    }
};

// |v| as a word: for values other than NaN these words order as the
// magnitudes do, and a word of 0x7F800000 or more is an infinity or a NaN, so
// one integer maximum gives both a group's amax and whether it fails.
NQ_HD uint32_t gq_mag(float v) { return __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu; }
constexpr uint32_t GQ_NONFINITE = 0x7F800000u;  // smallest magnitude word that fails
NQ_HD uint32_t gq_umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// clamp(x, lo, hi) for lo <= hi and x not NaN (v_med3_f32).
NQ_HD float gq_clamp(float x, float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_fmed3f(x, lo, hi);
#else
    return x < lo ? lo : x > hi ? hi : x;
#endif
}

// Code byte of a clamped quotient c (|c| <= 127): adding 1.5 * 2^23 leaves a
// sum in [2^23, 2^24), where binary32 spacing is 1, so the addition itself
// rounds c half to even and the sum's low mantissa byte is that integer in
// two's complement.
NQ_HD uint32_t gq_code_word(float c) { return __builtin_bit_cast(uint32_t, A(c, 12582912.0f)); }

// binary32 -> binary16 word, round-to-nearest-even (overflow gives infinity,
// subnormals are kept): the hardware conversion under the default mode.
NQ_HD uint32_t gq_f32_to_f16(float v) {
    f32x2 p;
    p.x = v;
    p.y = 0.0f;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2)) & 0xFFFFu;
}

// Group g (launch-relative) of lane-chunk j (values j*VPL .. j*VPL+VPL-1 of
// the group): the chunk's source offset from x, and how many of its values
// exist.
template <int GQ_VPL>
NQ_HD uint32_t gq_chunk(const GqArgs &a, int G, uint32_t g, uint32_t j, uint64_t *off) {
    const uint32_t r = (uint32_t)(((uint64_t)g * a.gmul) >> a.gshift);  // row, g / ngr
    const uint32_t col = (g - r * a.ngr) * (uint32_t)G + (uint32_t)GQ_VPL * j;
    *off = (uint64_t)r * a.K + col;
    return col >= a.K ? 0u : (a.K - col < (uint32_t)GQ_VPL ? a.K - col : (uint32_t)GQ_VPL);
}

// Phase 1: a lane's GQ_VPL source values (zeros past the group's end) and
// the largest of their magnitude words (gq_mag).
template <int IN, bool VECIN, class Src, int GQ_VPL = gq_vpl<IN>()>
NQ_HD uint32_t gq_load(const Src &src, uint64_t off, uint32_t cnt, float (&v)[GQ_VPL]) {
    if (VECIN && cnt == (uint32_t)GQ_VPL) {
        src.template span<IN>(off, v);
    } else {
        for (int k = 0; k < GQ_VPL; k++)
            v[k] = (uint32_t)k < cnt ? src.template one<IN>(off + (uint64_t)k) : 0.0f;
    }
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < GQ_VPL; k++) m = gq_umax(m, gq_mag(v[k]));
    return m;
}

// Phase 3: the group's scale word from its amax (every lane of the group
// computes it), and the lane's codes, four bytes to a word in value order.
// Returns status bits.  rint-then-clamp equals clamp-then-rint here because
// the bounds are integers and rounding is monotonic.
template <int S, int GQ_VPL>
NQ_HD uint32_t gq_encode(float amax, const float (&v)[GQ_VPL], uint32_t *s16_out, uint32_t (&qw)[GQ_VPL / 4]) {
    constexpr float qmin = (float)GQ[S].qmin, qmax = (float)GQ[S].qmax;
#pragma unroll
    for (int d = 0; d < GQ_VPL / 4; d++) qw[d] = 0u;
    if (amax == 0.0f) {
        *s16_out = 0u;
        return 0u;
    }
    const float raw = amax / qmax;  // correctly rounded binary32 division
    uint32_t s16 = gq_f32_to_f16(raw);
    if (s16 == 0u) s16 = 1u;  // 2^-24 underflow rescue
    *s16_out = s16;
    if ((s16 & 0x7C00u) == 0x7C00u) return 2u;
    const float inv = 1.0f / f16(s16);
#pragma unroll
    for (int d = 0; d < GQ_VPL / 4; d++) {
        uint32_t c[4];
#pragma unroll
        for (int k = 0; k < 4; k++) c[k] = gq_code_word(gq_clamp(M(v[4 * d + k], inv), qmin, qmax));
        qw[d] = perm(perm(c[3], c[2], 0x00000400u), perm(c[1], c[0], 0x00000400u), 0x05040100u);
    }
    return 0u;
}

// Phase 3 stores: the lane's codes (GQ_VPL bytes, or the cnt that exist) and,
// for the group's first lane, the scale word.
template <bool VECOUT, int GQ_VPL>
NQ_HD void gq_store(const GqArgs &a, uint64_t off, uint32_t cnt, const uint32_t (&qw)[GQ_VPL / 4], uint32_t g,
                    uint32_t j, uint32_t s16) {
    if (VECOUT && cnt == (uint32_t)GQ_VPL) {
        uint32_t *p = (uint32_t *)(a.codes + off);
        if constexpr (GQ_VPL == 4) {
            p[0] = qw[0];
        } else {
#pragma unroll
            for (int d = 0; d < GQ_VPL / 4; d += 2) {
                u32x2a4 v;
                v.x = qw[d];
                v.y = qw[d + 1];
                *(u32x2a4 *)(p + d) = v;
            }
        }
    } else {
        for (uint32_t k = 0; k < cnt; k++) a.codes[off + k] = (int8_t)bytek(qw[k / 4u], k % 4u);
    }
    if (j == 0u) a.scales[g] = (uint16_t)s16;
}

template <int S, int IN, bool VECIN, bool VECOUT>
__global__ __launch_bounds__(WG) void k_grouped_absmax(GqArgs a) {
    constexpr int G = GQ[S].G;
    constexpr int GQ_VPL = gq_vpl<IN>();
    constexpr uint32_t LPG = (uint32_t)(G / GQ_VPL);  // lanes per group
    const uint32_t lin = blockIdx.x * (uint32_t)WG + threadIdx.x;
    const uint32_t g = lin / LPG, j = lin % LPG;
    const bool live = g < a.ngroups;
    uint64_t off = 0;
    const uint32_t cnt = live ? gq_chunk<GQ_VPL>(a, G, g, j, &off) : 0u;
    float v[GQ_VPL];
    uint32_t mag = gq_load<IN, VECIN>(GqDevSrc{a.x}, off, cnt, v);
    // the group's lanes are consecutive: exchange within each run of LPG lanes
    // (max is exact, so the order of the exchange does not matter)
#pragma unroll
    for (uint32_t d = 1; d < LPG; d <<= 1) mag = gq_umax(mag, (uint32_t)__shfl_xor((int)mag, (int)d, 64));
    if (!live) return;
    uint32_t s16 = 0;
    uint32_t q[GQ_VPL / 4];
    const uint32_t st = mag >= GQ_NONFINITE ? 1u : gq_encode<S>(bits_f32(mag), v, &s16, q);
    if (st != 0u) {
        if (j == 0u) atomicOr(a.status, st);
        return;
    }
    gq_store<VECOUT, GQ_VPL>(a, off, cnt, q, g, j, s16);
}

// Host side: one matrix, split into launches of at most 2^30 groups.
struct GqLaunch {
    const void *x;
    int8_t *codes;
    uint16_t *scales;
    uint32_t *status;
    uint64_t N, K;
};

constexpr uint64_t GQ_CHUNK_GROUPS = 1ull << 30;  // groups per launch at most

// Arguments of the launch starting at row r0 (as many rows as fit the chunk
// limit), with its row count and grid size.
template <int S, int IN>
NQ_HD GqArgs gq_chunk_args(const GqLaunch &L, uint64_t r0, uint64_t *rows, uint32_t *grid) {
    constexpr uint64_t G = (uint64_t)GQ[S].G, LPG = G / (uint64_t)gq_vpl<IN>();
    constexpr uint64_t ESZ = IN == 0 ? 4 : IN == 3 ? 8 : 2;
    const uint64_t ngr = (L.K + G - 1) / G;
    const uint64_t per = GQ_CHUNK_GROUPS / ngr;  // ngr <= 2^26, so per >= 16
    *rows = L.N - r0 < per ? L.N - r0 : per;
    GqArgs a;
    a.x = (const uint8_t *)L.x + r0 * L.K * ESZ;
    a.codes = L.codes + r0 * L.K;
    a.scales = L.scales + r0 * ngr;
    a.status = L.status;
    a.K = (uint32_t)L.K;
    a.ngr = (uint32_t)ngr;
    a.ngroups = (uint32_t)(*rows * ngr);
    div_magic(ngr, &a.gmul, &a.gshift);
    *grid = (uint32_t)((a.ngroups * LPG + WG - 1) / WG);
    return a;
}

int launch_grouped_absmax(int scheme, int in_dtype, const GqLaunch &L, hipStream_t s);

}  // namespace nq
