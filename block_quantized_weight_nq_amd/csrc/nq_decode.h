// nq_decode.h -- per-format unit decoders for gfx950.
//
// A "unit" is 8 consecutive outputs j0 = 8s .. 8s+7 of one block (B is 32,
// 64, 128 or 256, so a block holds B/8 units).  Each decoder reads only the
// payload bytes its unit needs and evaluates the rule of the ONNX page
// "DequantizePacked decoding specification", section "Mathematical decoding
// rules", with the same binary32 operations in the same nesting: M, A and D
// are one IEEE multiply, add and subtract, compiled with -ffp-contract=off
// and fp32 denormals preserved.  Per-unit factors (sub-block scales, lane
// scales) are computed once per unit, never folded into a different product.
// "nvfp4" restates section 3.3 of the NInfer "tensor-formats" page.
//
// The decoders are __host__ __device__ and take their memory through a
// source type, so the same code runs in the kernels and in a host emulator
// that checks every access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define NQ_HD __host__ __device__ __forceinline__

namespace nq {

// Format ids: the order of the DequantizePacked page's identifier table,
// then "nvfp4".
enum Fmt : int {
    Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q8_1, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, Q8_K,
    IQ2_XXS, IQ2_XS, IQ3_XXS, IQ1_S, IQ4_NL, IQ3_S, IQ2_S, IQ4_XS, IQ1_M,
    TQ1_0, TQ2_0, MXFP4, NVFP4_GGUF, Q1_0, Q2_0, NVFP4_DIV, NUM_FORMATS
};

// Block geometry (B values, S bytes): "Quantization formats" table.
constexpr int block_values(int f) {
    return (f == Q4_0 || f == Q4_1 || f == Q5_0 || f == Q5_1 || f == Q8_0 || f == Q8_1 ||
            f == IQ4_NL || f == MXFP4) ? 32
         : (f == NVFP4_GGUF || f == NVFP4_DIV || f == Q2_0) ? 64
         : (f == Q1_0) ? 128 : 256;
}
constexpr int block_bytes(int f) {
    return f == Q4_0 ? 18 : f == Q4_1 ? 20 : f == Q5_0 ? 22 : f == Q5_1 ? 24 : f == Q8_0 ? 34
         : f == Q8_1 ? 36 : f == Q2_K ? 84 : f == Q3_K ? 110 : f == Q4_K ? 144 : f == Q5_K ? 176
         : f == Q6_K ? 210 : f == Q8_K ? 292 : f == IQ2_XXS ? 66 : f == IQ2_XS ? 74
         : f == IQ3_XXS ? 98 : f == IQ1_S ? 50 : f == IQ4_NL ? 18 : f == IQ3_S ? 110
         : f == IQ2_S ? 82 : f == IQ4_XS ? 136 : f == IQ1_M ? 56 : f == TQ1_0 ? 54
         : f == TQ2_0 ? 66 : f == MXFP4 ? 17 : f == NVFP4_GGUF ? 36 : f == Q1_0 ? 18
         : f == Q2_0 ? 18 : f == NVFP4_DIV ? 36 : 0;
}
constexpr bool is_iq(int f) {
    return f == IQ2_XXS || f == IQ2_XS || f == IQ2_S || f == IQ3_XXS || f == IQ3_S || f == IQ1_S ||
           f == IQ1_M;
}

// ---------------------------------------------------------------------------
// Bit helpers
// ---------------------------------------------------------------------------
// ({hi,lo} >> 8*sh)[31:0]: v_alignbyte_b32.
NQ_HD uint32_t alignbyte(uint32_t hi, uint32_t lo, uint32_t sh) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
#else
    return (uint32_t)(((((uint64_t)hi) << 32) | lo) >> (8u * (sh & 3u)));
#endif
}

// Byte select from the 8 bytes {hi,lo} with selectors 0..7 in each byte of
// sel (0-3 pick lo's bytes, 4-7 hi's): v_perm_b32.
NQ_HD uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(hi, lo, sel);
#else
    const uint64_t v = (((uint64_t)hi) << 32) | lo;
    uint32_t r = 0;
    for (int k = 0; k < 4; k++) {
        const uint32_t s = (sel >> (8 * k)) & 7u;
        r |= (uint32_t)((v >> (8 * s)) & 0xFFu) << (8 * k);
    }
    return r;
#endif
}

NQ_HD uint32_t bytek(uint32_t w, uint32_t k) { return (w >> (8u * k)) & 0xFFu; }

NQ_HD float bits_f32(uint32_t u) {
    float f;
    __builtin_memcpy(&f, &u, 4);
    return f;
}

// Exact binary16 -> binary32 (v_cvt_f32_f16; fp16 denormals are enabled).
NQ_HD float f16(uint32_t h) {
    const uint16_t hb = (uint16_t)h;
    _Float16 x;
    __builtin_memcpy(&x, &hb, 2);
    return (float)x;
}

// The page's binary32 operations.
NQ_HD float M(float a, float b) { return a * b; }
NQ_HD float A(float a, float b) { return a + b; }
NQ_HD float D(float a, float b) { return a - b; }

// 16-entry signed-byte table lookup for four 4-bit codes (one per byte of
// `codes`): t0..t3 hold entries 0-3, 4-7, 8-11, 12-15.
NQ_HD uint32_t lut16(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3, uint32_t codes) {
    const uint32_t lo3 = codes & 0x07070707u;
    const uint32_t a = perm(t1, t0, lo3);
    const uint32_t b = perm(t3, t2, lo3);
    const uint32_t m = ((codes >> 3) & 0x01010101u) * 0xFFu;
    return (b & m) | (a & ~m);
}
NQ_HD int sbyte(uint32_t w, uint32_t k) { return (int)(int8_t)(uint8_t)(w >> (8u * k)); }

// IQ4_NL table (Packed layouts section) as signed bytes, 4 per word.
constexpr uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
           ((uint32_t)(uint8_t)d << 24);
}
constexpr uint32_t IQ4T0 = pack4(-127, -104, -83, -65), IQ4T1 = pack4(-49, -35, -22, -10);
constexpr uint32_t IQ4T2 = pack4(1, 13, 25, 38), IQ4T3 = pack4(53, 69, 89, 113);
// Doubled E2M1 table V (both zero entries +0).
constexpr uint32_t FP4T0 = pack4(0, 1, 2, 3), FP4T1 = pack4(4, 6, 8, 12);
constexpr uint32_t FP4T2 = pack4(0, -1, -2, -3), FP4T3 = pack4(-4, -6, -8, -12);

// ---------------------------------------------------------------------------
// Payload windows.  `off` is a byte offset from the source's 4-byte-aligned
// base (32-bit: a launch covers less than 4 GiB of payload).  A window of ND
// dwords reads dwords a..a+ND-1 plus one more for the byte shift, through the
// source's dwx(): a global-memory source clamps that index to its last dword,
// so no access leaves the dwords that hold payload bytes, and an LDS source
// reads its padding.  Where that dword lies past the payload the shift is 0
// and the extra dword is not used.
template <int ND, class Src>
NQ_HD void window(const Src &src, uint32_t off, uint32_t (&w)[ND]) {
    const uint32_t a = off >> 2;
    const uint32_t sh = off & 3u;
    uint32_t r[ND];
    src.template load<ND>(a, r);
    const uint32_t extra = src.dwx(a + ND);
#pragma unroll
    for (int k = 0; k < ND; k++) w[k] = alignbyte(k + 1 < ND ? r[k + 1] : extra, r[k], sh);
}

template <class Src>
NQ_HD uint32_t u16_at(const Src &src, uint32_t off) {
    const uint32_t a = off >> 2;
    const uint32_t sh = off & 3u;
    const uint32_t r0 = src.dw(a);
    const uint32_t r1 = src.dwx(a + 1);
    return alignbyte(r1, r0, sh) & 0xFFFFu;
}

template <class Src>
NQ_HD uint32_t u8_at(const Src &src, uint32_t off) {
    return (src.dw(off >> 2) >> (8u * (off & 3u))) & 0xFFu;
}

// A value the compiler may not look through: code words built by a shift and
// a byte mask are then converted byte by byte (v_cvt_f32_ubyte0..3) instead of
// one bit-field extract per code.
NQ_HD uint32_t opaque(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm("" : "+v"(x));
#endif
    return x;
}

// 8 nibbles (plane `hi` of the 8 bytes in w[0], w[1]) as two words of 4 codes.
NQ_HD void nibbles(const uint32_t (&w)[2], uint32_t hi, uint32_t (&c)[2]) {
    c[0] = opaque((w[0] >> (4u * hi)) & 0x0F0F0F0Fu);
    c[1] = opaque((w[1] >> (4u * hi)) & 0x0F0F0F0Fu);
}
// 2-bit fields of plane p of the 8 bytes in w[0], w[1], one per byte.
NQ_HD void crumbs(const uint32_t (&w)[2], uint32_t p, uint32_t (&c)[2]) {
    c[0] = opaque((w[0] >> (2u * p)) & 0x03030303u);
    c[1] = opaque((w[1] >> (2u * p)) & 0x03030303u);
}
NQ_HD uint32_t code_at(const uint32_t (&c)[2], int k) { return bytek(c[k >> 2], (uint32_t)(k & 3)); }

// ---------------------------------------------------------------------------
// Unit decoders.  bo: byte offset of the block; s: unit index in the block.
// ---------------------------------------------------------------------------
struct NoTab {};

// Conventional formats: Q4_0, Q4_1, Q5_0, Q5_1, IQ4_NL (v = P(q,4,16)).
template <int F, class Src>
NQ_HD void unit_conventional(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    constexpr int QOFF = (F == Q4_0 || F == IQ4_NL) ? 2 : F == Q4_1 ? 4 : F == Q5_0 ? 6 : 8;
    uint32_t q[2];
    window<2>(src, bo + QOFF + 8u * (s & 1u), q);
    uint32_t c[2];
    nibbles(q, s >> 1, c);
    if constexpr (F == Q4_0 || F == IQ4_NL) {
        const float d = f16(u16_at(src, bo));
        if constexpr (F == Q4_0) {
#pragma unroll
            for (int k = 0; k < 8; k++) y[k] = M(d, (float)((int)code_at(c, k) - 8));
        } else {
            const uint32_t t[2] = {lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, c[0]),
                                   lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, c[1])};
#pragma unroll
            for (int k = 0; k < 8; k++) y[k] = M(d, (float)sbyte(t[k >> 2], (uint32_t)(k & 3)));
        }
    } else if constexpr (F == Q4_1) {
        uint32_t h[1];
        window<1>(src, bo, h);
        const float d = f16(h[0] & 0xFFFFu), m = f16(h[0] >> 16);
#pragma unroll
        for (int k = 0; k < 8; k++) y[k] = A(M(d, (float)code_at(c, k)), m);
    } else {
        // Q5_0: h d; u8 high[4] at 2.  Q5_1: h d,m; u8 high[4] at 4.
        uint32_t h[2];
        window<2>(src, bo, h);
        const float d = f16(h[0] & 0xFFFFu);
        const uint32_t high = (F == Q5_0) ? alignbyte(h[1], h[0], 2) : h[1];
        const uint32_t hb = (high >> (8u * s)) & 0xFFu;
        if constexpr (F == Q5_0) {
#pragma unroll
            for (int k = 0; k < 8; k++)
                y[k] = M(d, (float)((int)(code_at(c, k) + 16u * ((hb >> k) & 1u)) - 16));
        } else {
            const float m = f16(h[0] >> 16);
#pragma unroll
            for (int k = 0; k < 8; k++)
                y[k] = A(M(d, (float)(code_at(c, k) + 16u * ((hb >> k) & 1u))), m);
        }
    }
}

// Q8_0, Q8_1, Q8_K: y = M(d, q[j]); cached s / sums are never read.
template <int F, class Src>
NQ_HD void unit_q8(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    constexpr int QOFF = F == Q8_0 ? 2 : 4;
    float d;
    if constexpr (F == Q8_K) {
        uint32_t h[1];
        window<1>(src, bo, h);
        d = bits_f32(h[0]);
    } else {
        d = f16(u16_at(src, bo));
    }
    uint32_t q[2];
    window<2>(src, bo + QOFF + 8u * s, q);
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = M(d, (float)sbyte(q[k >> 2], (uint32_t)(k & 3)));
}

// Q1_0: y = d if bit set else -d (no rounding).
template <class Src>
NQ_HD void unit_q1_0(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    const float d = f16(u16_at(src, bo));
    const uint32_t b = u8_at(src, bo + 2 + s);
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = ((b >> k) & 1u) ? d : -d;
}

// Q2_0: v = P(q,2,1): byte t holds outputs 4t..4t+3; y = M(d, v-1).
template <class Src>
NQ_HD void unit_q2_0(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    const float d = f16(u16_at(src, bo));
    const uint32_t w = u16_at(src, bo + 2 + 2u * s);
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = M(d, (float)((int)((w >> (2 * k)) & 3u) - 1));
}

// Q2_K: v = P(q,2,32); s = scales[j/16]; y = D(M(M(d, s mod 16), v), M(dmin, s/16)).
template <class Src>
NQ_HD void unit_q2_k(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    uint32_t q[2];
    window<2>(src, bo + 16 + 32u * (s >> 4) + 8u * (s & 3u), q);
    uint32_t c[2];
    crumbs(q, (s >> 2) & 3u, c);
    const uint32_t sc = u8_at(src, bo + (s >> 1));
    uint32_t h[1];
    window<1>(src, bo + 80, h);
    const float d = f16(h[0] & 0xFFFFu), dmin = f16(h[0] >> 16);
    const float da = M(d, (float)(sc & 15u));
    const float dm = M(dmin, (float)(sc >> 4));
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = D(M(da, (float)code_at(c, k)), dm);
}

// Q3_K: v = P(q,2,32), h = P(mask,1,32), l = P(b[96:104],4,8),
// a = P(b[104:108],2,4); s = l[k] + 16 a[k] - 32; y = M(M(d,s), v - 4(1-h)).
template <class Src>
NQ_HD void unit_q3_k(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    uint32_t q[2], mk[2], sc[3];
    window<2>(src, bo + 32 + 32u * (s >> 4) + 8u * (s & 3u), q);
    window<2>(src, bo + 8u * (s & 3u), mk);
    window<3>(src, bo + 96, sc);
    const float d = f16(u16_at(src, bo + 108));
    uint32_t c[2];
    crumbs(q, (s >> 2) & 3u, c);
    const uint32_t hbit = s >> 2;
    const uint32_t k = s >> 1;
    const uint32_t lk = k & 7u;
    const uint32_t lbyte = bytek((lk < 4u) ? sc[0] : sc[1], lk & 3u);
    const uint32_t l = (lbyte >> (4u * (k >> 3))) & 15u;
    const uint32_t a = (bytek(sc[2], k & 3u) >> (2u * (k >> 2))) & 3u;
    const float ds = M(d, (float)((int)(l + 16u * a) - 32));
    // v - 4(1 - h) = (v + 4h) - 4: each byte takes its mask bit as bit 2
    // beside its 2-bit code (four values per operation)
    c[0] = opaque(c[0] | (((mk[0] >> hbit) & 0x01010101u) << 2));
    c[1] = opaque(c[1] | (((mk[1] >> hbit) & 0x01010101u) << 2));
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = M(ds, (float)code_at(c, j) - 4.0f);
}

// Q4_K / Q5_K: a[k], m[k] from the 12-byte scales; v = P(q,4,32) (+16 P(high,1,32));
// y = D(M(M(d,a[k]),v), M(dmin,m[k])), k = j/32.
template <int F, class Src>
NQ_HD void unit_q45_k(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    constexpr int QOFF = F == Q4_K ? 16 : 48;
    uint32_t hdr[4], q[2];
    window<4>(src, bo, hdr);
    window<2>(src, bo + QOFF + 32u * (s >> 3) + 8u * (s & 3u), q);
    const float d = f16(hdr[0] & 0xFFFFu), dmin = f16(hdr[0] >> 16);
    const uint32_t k = s >> 2, kk = k & 3u;
    const uint32_t b0 = bytek(hdr[1], kk), b1 = bytek(hdr[2], kk), b2 = bytek(hdr[3], kk);
    // k < 4: a = s[k] mod 64, m = s[k+4] mod 64; otherwise the 4+2-bit splits.
    const bool lo = k < 4u;
    const uint32_t a = lo ? (b0 & 63u) : ((b2 & 15u) | ((b0 >> 6) << 4));
    const uint32_t m = lo ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
    uint32_t c[2];
    nibbles(q, (s >> 2) & 1u, c);
    if constexpr (F == Q5_K) {
        uint32_t hi[2];
        window<2>(src, bo + 16 + 8u * (s & 3u), hi);
        const uint32_t sh = s >> 2;
        c[0] += ((hi[0] >> sh) & 0x01010101u) << 4;
        c[1] += ((hi[1] >> sh) & 0x01010101u) << 4;
    }
    const float da = M(d, (float)a);
    const float dm = M(dmin, (float)m);
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = D(M(da, (float)code_at(c, j)), dm);
}

// Q6_K: l = P(low,4,64), h = P(high,2,32), s = scales[j/16] (signed);
// y = M(M(d,s), l + 16h - 32).
template <class Src>
NQ_HD void unit_q6_k(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    uint32_t lw[2], hw[2];
    window<2>(src, bo + 64u * (s >> 4) + 8u * (s & 7u), lw);
    window<2>(src, bo + 128 + 32u * (s >> 4) + 8u * (s & 3u), hw);
    const int sc = (int)(int8_t)(uint8_t)u8_at(src, bo + 192 + (s >> 1));
    const float d = f16(u16_at(src, bo + 208));
    uint32_t lc[2], hc[2];
    nibbles(lw, (s >> 3) & 1u, lc);
    crumbs(hw, (s >> 2) & 3u, hc);
    const float ds = M(d, (float)sc);
#pragma unroll
    for (int j = 0; j < 8; j++)
        y[j] = M(ds, (float)((int)(code_at(lc, j) + 16u * code_at(hc, j)) - 32));
}

// IQ4_XS: s[k] = field(scales[k/2], 4(k mod 2), 4) + 16 field(high, 2k, 2) - 32;
// y = M(M(d, s[j/32]), IQ4[v]), v = P(q,4,16).
template <class Src>
NQ_HD void unit_iq4_xs(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    uint32_t hdr[2], q[2];
    window<2>(src, bo, hdr);
    window<2>(src, bo + 8 + 16u * (s >> 2) + 8u * (s & 1u), q);
    const float d = f16(hdr[0] & 0xFFFFu);
    const uint32_t high = hdr[0] >> 16;
    const uint32_t k = s >> 2;
    const uint32_t lo = (bytek(hdr[1], k >> 1) >> (4u * (k & 1u))) & 15u;
    const uint32_t sk = lo + 16u * ((high >> (2u * k)) & 3u);
    const float ds = M(d, (float)((int)sk - 32));
    uint32_t c[2];
    nibbles(q, (s >> 1) & 1u, c);
    const uint32_t t[2] = {lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, c[0]), lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, c[1])};
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = M(ds, (float)sbyte(t[j >> 2], (uint32_t)(j & 3)));
}

// Q8_K: f d; i8 q[256].
// (handled by unit_q8<Q8_K>)

// TQ1_0: sequences (0,32,5), (32,16,5), (48,4,4); t = floor(3((b 3^p) mod 256)/256) - 1.
NQ_HD uint32_t pow3(uint32_t p) { return p == 0 ? 1u : p == 1 ? 3u : p == 2 ? 9u : p == 3 ? 27u : 81u; }

// Digit k of each byte of w (byte b of the result: floor(3 * ((byte * 3^k)
// mod 256) / 256), 0..2), two bytes per multiply in 16-bit fields: byte *
// 3^k <= 20655 and 3 * 255 stay inside a field.
// With m = 3^k given: bytes 0 and 2, and bytes 1 and 3, are moved into the
// low bytes of two 16-bit fields by byte selects; after the multiply and the
// mod-256 mask, 3 * r leaves each digit in bits 8-9 of its field, and one
// more byte select gathers the four digits in byte order.
NQ_HD uint32_t digits4m(uint32_t w, uint32_t m) {
    const uint32_t e = perm(0u, w, 0x04020400u);  // [b0, 0, b2, 0]
    const uint32_t o = perm(0u, w, 0x04030401u);  // [b1, 0, b3, 0]
    const uint32_t fe = ((e * m) & 0x00FF00FFu) * 3u & 0x03000300u;
    const uint32_t fo = ((o * m) & 0x00FF00FFu) * 3u & 0x03000300u;
    return perm(fo, fe, 0x07030501u);  // [fe byte 1, fo byte 1, fe byte 3, fo byte 3]
}

NQ_HD uint32_t digits4(uint32_t w, uint32_t k) { return digits4m(w, pow3(k)); }

// Unit s of a tq1_0 block, without branches (a wave's lanes hold every s):
// s < 20 takes digit s/4 of bytes 8(s mod 4) .. +7; 20 <= s < 30 digit
// (s-20)/2 of bytes 32 + 8((s-20) mod 2) .. +7; s >= 30 digits 2(s-30) and
// 2(s-30)+1 of bytes 48..51 (outputs 240 + 4k + i: digit k of byte 48 + i).
// One 8-byte window per unit (at 44 for s >= 30, whose upper half holds
// bytes 48..51); y = M(d, digit - 1).
template <class Src>
NQ_HD void unit_tq1_0(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    const float d = f16(u16_at(src, bo + 52));
    const bool first = s < 20u, tail = s >= 30u;
    const uint32_t off = first ? 8u * (s & 3u) : tail ? 44u : 32u + 8u * ((s - 20u) & 1u);
    const uint32_t p0 = first ? s >> 2 : tail ? 2u * (s - 30u) : (s - 20u) >> 1;
    uint32_t q[2];
    window<2>(src, bo + off, q);
    uint32_t c[2];
    c[0] = opaque(digits4(tail ? q[1] : q[0], p0));
    c[1] = opaque(digits4(q[1], tail ? p0 + 1u : p0));
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = M(d, (float)code_at(c, j) - 1.0f);
}

// TQ2_0: y = M(d, v-1), v = P(q,2,32).
template <class Src>
NQ_HD void unit_tq2_0(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    uint32_t q[2];
    window<2>(src, bo + 32u * (s >> 4) + 8u * (s & 3u), q);
    uint32_t c[2];
    crumbs(q, (s >> 2) & 3u, c);
    const float d = f16(u16_at(src, bo + 64));
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = M(d, (float)((int)code_at(c, j) - 1));
}

// MXFP4: half scale bits 0x00200000 << e (e < 2) or (e-1) << 23; y = M(d, V[v]).
template <class Src>
NQ_HD void unit_mxfp4(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    const uint32_t e = u8_at(src, bo);
    uint32_t q[2];
    window<2>(src, bo + 1 + 8u * (s & 1u), q);
    const float d = bits_f32(e < 2u ? (0x00200000u << e) : ((e - 1u) << 23));
    uint32_t c[2];
    nibbles(q, s >> 1, c);
    const uint32_t t[2] = {lut16(FP4T0, FP4T1, FP4T2, FP4T3, c[0]), lut16(FP4T0, FP4T1, FP4T2, FP4T3, c[1])};
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = M(d, (float)sbyte(t[j >> 2], (uint32_t)(j & 3)));
}

// gguf:nvfp4 half scale: 0 for the whole byte 0 or 127; m 2^-10 for E = 0;
// (1 + m/8) 2^(E-8) otherwise; bit 7 enters neither E nor m.
NQ_HD float nvfp4_half_scale(uint32_t e) {
    const uint32_t E = (e >> 3) & 15u, m = e & 7u;
    if (e == 0u || e == 127u) return 0.0f;
    if (E == 0u) return M((float)m, 0x1p-10f);
    return bits_f32(((E + 119u) << 23) | (m << 20));
}

template <class Src>
NQ_HD void unit_nvfp4_gguf(const Src &src, uint32_t bo, uint32_t s, float (&y)[8]) {
    const uint32_t g = s >> 1;
    const float d = nvfp4_half_scale(u8_at(src, bo + g));
    uint32_t q[2];
    window<2>(src, bo + 4 + 8u * g, q);
    uint32_t c[2];
    nibbles(q, s & 1u, c);
    const uint32_t t[2] = {lut16(FP4T0, FP4T1, FP4T2, FP4T3, c[0]), lut16(FP4T0, FP4T1, FP4T2, FP4T3, c[1])};
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = M(d, (float)sbyte(t[j >> 2], (uint32_t)(j & 3)));
}

// nvfp4 (NInfer 3.3): y = RN32(e2m1(c) * e4m3fn(s) / d_w).  The product is
// exact in binary32, so the value is one correctly rounded division.  IEEE
// products and quotients take the XOR of their operands' signs (zeros
// included) and round symmetrically, so y is the quotient of the magnitudes
// with sign bit (c bit 3) ^ (s bit 7) ^ (d_w's sign).  The kernels read that
// magnitude from a per-workgroup table of all 128 x 8 (s & 0x7F, c & 7)
// quotients |e2m1_e4m3_div| and insert the sign bit (a NaN quotient stays a
// NaN whatever its sign).
NQ_HD float e4m3fn(uint32_t w) {
    const uint32_t sign = (w >> 7) & 1u, E = (w >> 3) & 15u, m = w & 7u;
    float mag;
    if (E == 0u)
        mag = M((float)m, 0x1p-9f);
    else if (E == 15u && m == 7u)
        mag = bits_f32(0x7FC00000u);
    else
        mag = bits_f32(((E + 120u) << 23) | (m << 20));
    return sign ? -mag : mag;
}
NQ_HD float e2m1(uint32_t c) {
    const uint32_t dbl = bytek(perm(FP4T1, FP4T0, c & 7u), 0);  // doubled magnitude 0..12
    const float mag = M((float)dbl, 0.5f);
    return (c & 8u) ? -mag : mag;
}
NQ_HD float e2m1_e4m3_div(uint32_t sw, uint32_t c, float dw) { return M(e2m1(c), e4m3fn(sw)) / dw; }

// Table entry k = 8 * (s & 0x7F) + (c & 7): the quotient's magnitude bits.
NQ_HD uint32_t nvfp4_table_entry(uint32_t k, float dw) {
    return __builtin_bit_cast(uint32_t, e2m1_e4m3_div(k >> 3, k & 7u, dw)) & 0x7FFFFFFFu;
}

// Four table entries of scale magnitude sm (0..127) from one division:
// class 0 fills codes 1, 2, 4, 6 (E2M1 0.5, 1, 2, 4 times the scale), class 1
// codes 0, 3, 5, 7 (0, 1.5, 3, 6).  With q = RN32(m * s / d_w) for m = 1 or
// 1.5, the entries are q/2, q, 2q, 4q (and 0 * s / d_w): scaling by a power
// of two is exact and commutes with round-to-nearest while neither side is
// subnormal, and an overflow of 2q or 4q to infinity happens on both sides
// alike.  So when q is finite and at least 2^-125 (q/2 still normal) the
// entries are scaled from q; otherwise (a q that overflowed, NaN, tiny or
// zero: only divisors that section 3.3 refuses, or a zero scale) each is
// divided directly.  Every entry equals nvfp4_table_entry.
NQ_HD void nvfp4_table_quad(uint32_t sm, uint32_t cls, float dw, uint32_t (&e)[4], uint32_t (&code)[4]) {
    code[0] = cls ? 0u : 1u;
    code[1] = cls ? 3u : 2u;
    code[2] = cls ? 5u : 4u;
    code[3] = cls ? 7u : 6u;
    const float q = e2m1_e4m3_div(sm, code[1], dw);  // E2M1 codes 2 (1.0) and 3 (1.5)
    const uint32_t b = __builtin_bit_cast(uint32_t, q) & 0x7FFFFFFFu;
    if (b >= 0x01000000u && b < 0x7F800000u) {
        const float a = bits_f32(b);
        // q finite: s is not the NaN word and d_w is neither NaN nor zero, so 0 * s / d_w is zero
        e[0] = cls ? 0u : __builtin_bit_cast(uint32_t, M(a, 0.5f));
        e[1] = b;
        e[2] = __builtin_bit_cast(uint32_t, M(a, 2.0f));
        e[3] = __builtin_bit_cast(uint32_t, M(a, 4.0f));
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) e[i] = nvfp4_table_entry(8u * sm + code[i], dw);
    }
}

// DIRECT: divide by `dw` here (the quotient carries d_w's sign; the codes'
// and scale's signs are XORed in) instead of reading the table built for the
// tile's first divisor group, whose magnitudes take the sign bit of all
// three (tab.nv_dsign: d_w's sign in bit 7 of every byte).  The same
// correctly rounded quotient either way.
template <bool DIRECT, class Src, class Tab>
NQ_HD void unit_nvfp4_div(const Src &src, uint32_t bo, uint32_t s, const Tab &tab, float dw, float (&y)[8]) {
    const uint32_t g = s >> 1;
    const uint32_t sw = u8_at(src, bo + g);
    uint32_t q[2];
    window<2>(src, bo + 4 + 8u * g, q);
    uint32_t c[2];
    nibbles(q, s & 1u, c);
    if constexpr (DIRECT) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t code = code_at(c, j);
            const uint32_t neg = ((code >> 3) ^ (sw >> 7)) & 1u;
            const float v = e2m1_e4m3_div(sw & 0x7Fu, code & 7u, dw);
            y[j] = bits_f32(__builtin_bit_cast(uint32_t, v) ^ (neg << 31));
        }
    } else {
        // per byte: the sign (bit 7) and the table offset in bytes (4 * code magnitude)
        const uint32_t sm = ((sw & 0x80u) ? 0x80808080u : 0u) ^ tab.nv_dsign;
        const uint32_t sg[2] = {((c[0] << 4) & 0x80808080u) ^ sm, ((c[1] << 4) & 0x80808080u) ^ sm};
        const uint32_t ix[2] = {opaque((c[0] & 0x07070707u) << 2), opaque((c[1] & 0x07070707u) << 2)};
        const uint32_t row = 32u * (sw & 0x7Fu);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t mag = tab.nvb(row + code_at(ix, j));
            const uint32_t sbit = sg[j >> 2] << (24 - 8 * (j & 3));
            y[j] = bits_f32((mag & 0x7FFFFFFFu) | (sbit & 0x80000000u));
        }
    }
}

// --- IQ2 / IQ3 / IQ1: unit = lane i = 4g + l --------------------------------
NQ_HD uint32_t parity7(uint32_t v) { return (uint32_t)__builtin_popcount(v & 127u) & 1u; }

template <int F, class Src, class Tab>
NQ_HD void unit_iq(const Src &src, uint32_t bo, uint32_t i, const Tab &tab, float (&y)[8]) {
    const uint32_t g = i >> 2, l = i & 3u;
    if constexpr (F == IQ1_S || F == IQ1_M) {
        float d, c, delta;
        uint32_t r;
        if constexpr (F == IQ1_S) {
            d = f16(u16_at(src, bo));
            const uint32_t lo = u8_at(src, bo + 2 + i);
            const uint32_t a = u16_at(src, bo + 34 + 2u * g);
            r = lo | (((a >> (3u * l)) & 7u) << 8);
            c = M(d, (float)(2u * ((a >> 12) & 7u) + 1u));
            delta = (a & 0x8000u) ? -0.125f : 0.125f;
        } else {
            uint32_t w[2];
            window<2>(src, bo + 48, w);
            const uint32_t dbits = (((w[0] & 0xFFFFu) >> 12)) | ((w[0] >> 28) << 4) |
                                   (((w[1] & 0xFFFFu) >> 12) << 8) | ((w[1] >> 28) << 12);
            d = f16(dbits);
            const uint32_t lo = u8_at(src, bo + i);
            const uint32_t a = (u8_at(src, bo + 32 + (i >> 1)) >> (4u * (i & 1u))) & 15u;
            r = lo | ((a & 7u) << 8);
            const uint32_t kw = g >> 1;  // scale word w[kw]: dword kw/2, half kw%2
            const uint32_t wg = ((kw >> 1) == 0u ? w[0] : w[1]) >> (16u * (kw & 1u));
            const uint32_t t = (wg >> (6u * (g & 1u) + 3u * (l >> 1))) & 7u;
            c = M(d, (float)(2u * t + 1u));
            delta = (a & 8u) ? -0.125f : 0.125f;
        }
        const uint64_t row = tab.iq1s(r);  // byte j = value j + 1
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int v = (int)((row >> (8 * j)) & 0xFFu) - 1;
            y[j] = M(c, A((float)v, delta));
        }
    } else {
        float c;
        uint32_t signs;
        uint32_t v[8];
        const float d = f16(u16_at(src, bo));
        if constexpr (F == IQ2_XXS) {
            uint32_t w[2];
            window<2>(src, bo + 2 + 8u * g, w);
            const uint32_t idx = bytek(w[0], l);
            const uint32_t aux = w[1];
            const uint32_t s7 = (aux >> (7u * l)) & 127u;
            signs = s7 | (parity7(s7) << 7);
            c = M(M(d, A(0.5f, (float)(aux >> 28))), 0.25f);
            const uint64_t row = tab.iq2xxs(idx);
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = (uint32_t)(row >> (8 * j)) & 0xFFu;
        } else if constexpr (F == IQ2_XS) {
            const uint32_t word = u16_at(src, bo + 2 + 2u * i);
            const uint32_t t = (u8_at(src, bo + 66 + g) >> (4u * (l >> 1))) & 15u;
            const uint32_t s7 = word >> 9;
            signs = s7 | (parity7(s7) << 7);
            c = M(M(d, A(0.5f, (float)t)), 0.25f);
            const uint64_t row = tab.iq2xs(word & 511u);
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = (uint32_t)(row >> (8 * j)) & 0xFFu;
        } else if constexpr (F == IQ2_S) {
            const uint32_t lo = u8_at(src, bo + 2 + i);
            signs = u8_at(src, bo + 34 + i);
            const uint32_t hi = (u8_at(src, bo + 66 + g) >> (2u * l)) & 3u;
            const uint32_t t = (u8_at(src, bo + 74 + g) >> (4u * (l >> 1))) & 15u;
            c = M(M(d, A(0.5f, (float)t)), 0.25f);
            const uint64_t row = tab.iq2s(lo | (hi << 8));
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = (uint32_t)(row >> (8 * j)) & 0xFFu;
        } else if constexpr (F == IQ3_XXS) {
            const uint32_t idx2 = u16_at(src, bo + 2 + 2u * i);
            uint32_t aw[1];
            window<1>(src, bo + 66 + 4u * g, aw);
            const uint32_t aux = aw[0];
            const uint32_t s7 = (aux >> (7u * l)) & 127u;
            signs = s7 | (parity7(s7) << 7);
            c = M(M(d, A(0.5f, (float)(aux >> 28))), 0.5f);
            const uint32_t r0 = tab.iq3xxs(idx2 & 0xFFu), r1 = tab.iq3xxs(idx2 >> 8);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[j] = (r0 >> (8 * j)) & 0xFFu;
                v[4 + j] = (r1 >> (8 * j)) & 0xFFu;
            }
        } else {  // IQ3_S
            const uint32_t idx2 = u16_at(src, bo + 2 + 2u * i);
            const uint32_t h = u8_at(src, bo + 66 + g);
            signs = u8_at(src, bo + 74 + i);
            const uint32_t sc = u8_at(src, bo + 106 + (g >> 1));
            c = M(d, (float)(1u + 2u * ((sc >> (4u * (g & 1u))) & 15u)));
            const uint32_t i0 = (idx2 & 0xFFu) | (((h >> (2u * l)) & 1u) << 8);
            const uint32_t i1 = (idx2 >> 8) | (((h >> (2u * l + 1u)) & 1u) << 8);
            const uint32_t r0 = tab.iq3s(i0), r1 = tab.iq3s(i1);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[j] = (r0 >> (8 * j)) & 0xFFu;
                v[4 + j] = (r1 >> (8 * j)) & 0xFFu;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float sj = ((signs >> j) & 1u) ? -1.0f : 1.0f;
            y[j] = M(M(c, (float)v[j]), sj);
        }
    }
}

// Dispatch one unit of format F.
template <int F, class Src, class Tab>
NQ_HD void decode_unit(const Src &src, uint32_t bo, uint32_t s, const Tab &tab, float (&y)[8]) {
    if constexpr (F == Q4_0 || F == Q4_1 || F == Q5_0 || F == Q5_1 || F == IQ4_NL)
        unit_conventional<F>(src, bo, s, y);
    else if constexpr (F == Q8_0 || F == Q8_1 || F == Q8_K)
        unit_q8<F>(src, bo, s, y);
    else if constexpr (F == Q1_0)
        unit_q1_0(src, bo, s, y);
    else if constexpr (F == Q2_0)
        unit_q2_0(src, bo, s, y);
    else if constexpr (F == Q2_K)
        unit_q2_k(src, bo, s, y);
    else if constexpr (F == Q3_K)
        unit_q3_k(src, bo, s, y);
    else if constexpr (F == Q4_K || F == Q5_K)
        unit_q45_k<F>(src, bo, s, y);
    else if constexpr (F == Q6_K)
        unit_q6_k(src, bo, s, y);
    else if constexpr (F == IQ4_XS)
        unit_iq4_xs(src, bo, s, y);
    else if constexpr (F == TQ1_0)
        unit_tq1_0(src, bo, s, y);
    else if constexpr (F == TQ2_0)
        unit_tq2_0(src, bo, s, y);
    else if constexpr (F == MXFP4)
        unit_mxfp4(src, bo, s, y);
    else if constexpr (F == NVFP4_GGUF)
        unit_nvfp4_gguf(src, bo, s, y);
    else if constexpr (F == NVFP4_DIV)
        unit_nvfp4_div<false>(src, bo, s, tab, 0.0f, y);
    else
        unit_iq<F>(src, bo, s, tab, y);
}

}  // namespace nq
