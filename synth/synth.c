/*
 * synth.c -- seeded synthetic payload generator for packed block-quantized
 * weights.  It knows only where each format keeps its scale fields (the
 * byte layout), never how a block decodes: it holds none of the decode
 * arithmetic, and both the HIP path's tests/benchmark and the oracle's tests
 * take their inputs from it.
 *
 * Random numbers: counter-based SplitMix64 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014; the
 * 64-bit finaliser with constants 0xbf58476d1ce4e5b9 and 0x94d049bb133111eb
 * and increment 0x9e3779b97f4a7c15).  Word k of block b for seed s is
 * mix(mix(s) + (64*b + k + 1) * GAMMA), so every block is a pure function
 * of (seed, block) and blocks fill in parallel.
 *
 * Modes:
 *   0 raw     every byte uniform (all scale encodings: zeros, subnormals,
 *             infinities, NaNs, negative values);
 *   1 recipe  bytes uniform except the scale fields, which follow the
 *             workload recipe: binary16 scales log-uniform over whole binades
 *             [2^lo, 2^hi) (random binade, uniform 10-bit fraction), with a
 *             random sign when `signed_scales`; binary32 scales likewise with
 *             a 23-bit fraction; E8M0 exponent bytes uniform in [118, 130];
 *             unsigned-E4M3 / E4M3FN block scale bytes uniform in [0x01,0x7E];
 *             ternary 2-bit codes uniform in {0,1,2} (tq2_0); the iq1_m
 *             binary16 scale scattered into the top nibbles of its four
 *             scale words with the low 12 bits uniform.
 */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ull

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static inline uint64_t word(uint64_t key, uint64_t block, unsigned k)
{
    return mix64(key + (64ull * block + (uint64_t)k + 1ull) * GAMMA);
}

uint64_t synth_splitmix64(uint64_t seed, uint64_t block, unsigned k)
{
    return word(mix64(seed), block, k);
}

/* Layout kinds of special fields. */
enum { K_F16 = 1, K_F32, K_E8M0, K_E4M3x4, K_TERN2x64, K_IQ1M };

typedef struct {
    const char *name;
    int S;          /* bytes per block */
    int trailer;    /* bytes after the last block */
    int nfields;
    struct { int kind, offset; } f[3];
} layout;

/* Scale field positions from the packed-layout table (fields concatenated
 * from byte 0 in the order listed there). */
static const layout LAYOUTS[] = {
    {"gguf:q4_0", 18, 0, 1, {{K_F16, 0}}},
    {"gguf:q4_1", 20, 0, 2, {{K_F16, 0}, {K_F16, 2}}},
    {"gguf:q5_0", 22, 0, 1, {{K_F16, 0}}},
    {"gguf:q5_1", 24, 0, 2, {{K_F16, 0}, {K_F16, 2}}},
    {"gguf:q8_0", 34, 0, 1, {{K_F16, 0}}},
    {"gguf:q8_1", 36, 0, 2, {{K_F16, 0}, {K_F16, 2}}},
    {"gguf:q2_k", 84, 0, 2, {{K_F16, 80}, {K_F16, 82}}},
    {"gguf:q3_k", 110, 0, 1, {{K_F16, 108}}},
    {"gguf:q4_k", 144, 0, 2, {{K_F16, 0}, {K_F16, 2}}},
    {"gguf:q5_k", 176, 0, 2, {{K_F16, 0}, {K_F16, 2}}},
    {"gguf:q6_k", 210, 0, 1, {{K_F16, 208}}},
    {"gguf:q8_k", 292, 0, 1, {{K_F32, 0}}},
    {"gguf:iq2_xxs", 66, 0, 1, {{K_F16, 0}}},
    {"gguf:iq2_xs", 74, 0, 1, {{K_F16, 0}}},
    {"gguf:iq3_xxs", 98, 0, 1, {{K_F16, 0}}},
    {"gguf:iq1_s", 50, 0, 1, {{K_F16, 0}}},
    {"gguf:iq4_nl", 18, 0, 1, {{K_F16, 0}}},
    {"gguf:iq3_s", 110, 0, 1, {{K_F16, 0}}},
    {"gguf:iq2_s", 82, 0, 1, {{K_F16, 0}}},
    {"gguf:iq4_xs", 136, 0, 1, {{K_F16, 0}}},
    {"gguf:iq1_m", 56, 0, 1, {{K_IQ1M, 48}}},
    {"gguf:tq1_0", 54, 0, 1, {{K_F16, 52}}},
    {"gguf:tq2_0", 66, 0, 2, {{K_TERN2x64, 0}, {K_F16, 64}}},
    {"gguf:mxfp4", 17, 0, 1, {{K_E8M0, 0}}},
    {"gguf:nvfp4", 36, 0, 1, {{K_E4M3x4, 0}}},
    {"gguf:q1_0", 18, 0, 1, {{K_F16, 0}}},
    {"gguf:q2_0", 18, 0, 1, {{K_F16, 0}}},
    {"nvfp4", 36, 4, 1, {{K_E4M3x4, 0}}},
};
#define NLAYOUTS ((int)(sizeof(LAYOUTS) / sizeof(LAYOUTS[0])))

static const layout *find(const char *name)
{
    for (int i = 0; i < NLAYOUTS; i++)
        if (strcmp(LAYOUTS[i].name, name) == 0) return &LAYOUTS[i];
    return 0;
}

int synth_block_bytes(const char *name)
{
    const layout *L = find(name);
    return L ? L->S : -1;
}

int synth_trailer_bytes(const char *name)
{
    const layout *L = find(name);
    return L ? L->trailer : -1;
}

static uint16_t f16_binade(uint64_t r, int lo, int hi, int signed_scales)
{
    const unsigned span = (unsigned)(hi - lo);
    const unsigned e = (unsigned)(lo + 15) + (unsigned)(r % span); /* biased exponent */
    const unsigned frac = (unsigned)((r >> 20) & 1023u);
    const unsigned sign = signed_scales ? (unsigned)((r >> 40) & 1u) : 0u;
    return (uint16_t)((sign << 15) | (e << 10) | frac);
}

static uint32_t f32_binade(uint64_t r, int lo, int hi, int signed_scales)
{
    const unsigned span = (unsigned)(hi - lo);
    const unsigned e = (unsigned)(lo + 127) + (unsigned)(r % span);
    const uint32_t frac = (uint32_t)((r >> 16) & 0x7FFFFFu);
    const uint32_t sign = signed_scales ? (uint32_t)((r >> 50) & 1u) : 0u;
    return (sign << 31) | (e << 23) | frac;
}

static void put16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }

static void fill_block(const layout *L, uint64_t key, uint64_t blk, int mode, int lo, int hi,
                       int signed_scales, uint8_t *b)
{
    /* words 0..36 carry the raw bytes (S <= 292) */
    for (int k = 0; 8 * k < L->S; k++) {
        const uint64_t w = word(key, blk, (unsigned)k);
        for (int i = 0; i < 8 && 8 * k + i < L->S; i++) b[8 * k + i] = (uint8_t)(w >> (8 * i));
    }
    if (mode == 0) return;
    for (int fi = 0; fi < L->nfields; fi++) {
        const int kind = L->f[fi].kind, off = L->f[fi].offset;
        const uint64_t r = word(key, blk, (unsigned)(48 + fi));
        switch (kind) {
        case K_F16: put16(b + off, f16_binade(r, lo, hi, signed_scales)); break;
        case K_F32: put32(b + off, f32_binade(r, lo, hi, signed_scales)); break;
        case K_E8M0: b[off] = (uint8_t)(118u + (unsigned)(r % 13u)); break;
        case K_E4M3x4:
            for (int g = 0; g < 4; g++) b[off + g] = (uint8_t)(1u + (unsigned)(((r >> (16 * g)) & 0xFFFFu) % 126u));
            break;
        case K_TERN2x64:
            /* 256 two-bit codes, each uniform in {0,1,2}, from words 16..47 */
            for (int byte = 0; byte < 64; byte++) {
                unsigned v = 0;
                for (int c = 0; c < 4; c++) {
                    const int code = 4 * byte + c;
                    const uint64_t w = word(key, blk, (unsigned)(16 + code / 8));
                    v |= (unsigned)(((w >> (8 * (code % 8))) & 0xFFu) % 3u) << (2 * c);
                }
                b[off + byte] = (uint8_t)v;
            }
            break;
        case K_IQ1M: {
            const uint16_t d = f16_binade(r, lo, hi, signed_scales);
            const uint64_t low = word(key, blk, 60);
            for (int k = 0; k < 4; k++) {
                const unsigned w = (unsigned)((low >> (12 * k)) & 0xFFFu) | ((unsigned)((d >> (4 * k)) & 15u) << 12);
                put16(b + off + 2 * k, (uint16_t)w);
            }
            break;
        }
        default: break;
        }
    }
}

/* Fill `nblocks` blocks of format `name` into out (nblocks * S bytes).
 * Returns 0, or -1 for an unknown name or a bad binade range. */
int synth_fill(const char *name, uint64_t nblocks, uint64_t seed, int mode, int lo, int hi,
               int signed_scales, uint8_t *out)
{
    const layout *L = find(name);
    if (!L || (mode == 1 && hi <= lo)) return -1;
    const uint64_t key = mix64(seed);
    const int64_t n = (int64_t)nblocks;
#pragma omp parallel for schedule(static, 4096)
    for (int64_t i = 0; i < n; i++)
        fill_block(L, key, (uint64_t)i, mode, lo, hi, signed_scales, out + (uint64_t)i * (uint64_t)L->S);
    return 0;
}

/* A binary32 divisor with bits uniform in [bits(1.0), bits(448.0)]. */
uint32_t synth_divisor_bits(uint64_t seed)
{
    const uint32_t lo = 0x3F800000u, hi = 0x43E00000u;
    return lo + (uint32_t)(mix64(mix64(seed) ^ 0x5eed) % (uint64_t)(hi - lo + 1u));
}
