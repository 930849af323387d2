// nq_gemv.h -- products of packed gguf_* weights with q8_1 activations.
//
// NInfer "tensor-formats" page: a product over a gguf_* weight quantizes the
// activation to ggml q8_1 numbers (one binary16 scale and one sum per 32
// values) and accumulates in FP32; the reduction order, staging and
// intermediate precision are the kernel's, and the observable result is
// judged against an independent oracle under a named criterion.
//
// Activation quantizer: for each 32 consecutive values of an activation row,
// the codes and the scale d follow the 8-bit, 32-value absmax rule of section
// 7.2 (q8_g32_fp16: amax, d = RN16(RN32(amax / 127)) with the 0x0001 rescue,
// inv = RN32(1 / d32), code = round-half-even(RN32(x * inv)) clamped to
// [-127, 127]); the sum field is RN16(d32 * sum of codes), a product that is
// exact in binary32.  Output: gguf q8_1 blocks (36 bytes: d, sum, 32 codes).
//
// Product: y[m][n] = sum_k w[n][k] * d[m][k/32] * q[m][k] for weight rows n
// and activation rows m < M <= 8, accumulated in binary32.  A wave owns a
// weight row: it stages the row's bytes in LDS, its 64 lanes take the row's
// items in turn and keep one FP32 partial per activation row, and the
// partials then meet in a fixed cross-lane tree, so every run gives the same
// bits.  Every gguf format takes integer items: its weights become 8-bit
// integers whose exact dot products with the activation codes are scaled in
// binary32 (the decoded-unit path below remains for formats without one).
#pragma once

#include <type_traits>

#include "nq_gqenc.h"

namespace nq {

constexpr int GV_MAX_M = 8;

// Signed 4 x 8-bit dot product with accumulation (v_dot4 on the GPU).
NQ_HD int dot4(uint32_t a, uint32_t b, int c) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
#else
    for (int k = 0; k < 4; k++) c += (int)(int8_t)(a >> (8 * k)) * (int)(int8_t)(b >> (8 * k));
    return c;
#endif
}

// ---------------------------------------------------------------- quantizer

// Blocks per quantizer launch: thread indices stay below 2^31.
constexpr uint64_t Q81_CHUNK = 1ull << 26;

struct Q81Args {
    const void *x;      // first source value of this launch
    uint32_t *blocks;   // its first q8_1 block (9 dwords per block)
    uint32_t *status;   // bit 0: non-finite source, 1: scale past binary16, 2: sum past binary16
    uint32_t nblocks;   // blocks in this launch
};

// Lanes per block: a lane takes gq_vpl<IN>() consecutive values (32 source
// bytes), so 4 (binary32), 2 (16-bit) or 8 (binary64) lanes share a block;
// they are adjacent lanes of one wave.
template <int IN>
constexpr uint32_t q81_lanes() {
    return 32u / (uint32_t)gq_vpl<IN>();
}

// Phase 2 of a lane (after the magnitude word is combined over the block's
// lanes): the block's d word, the lane's codes (four to a word; zero when the
// block fails) and status bits 0 and 1.
template <int VPL>
NQ_HD uint32_t q81_encode(uint32_t mag, const float (&v)[VPL], uint32_t *d16, uint32_t (&qw)[VPL / 4]) {
    uint32_t st = 1u;
    if (mag < GQ_NONFINITE) st = gq_encode<3, VPL>(bits_f32(mag), v, d16, qw);
    if (st) {
        *d16 = 0u;
#pragma unroll
        for (int d = 0; d < VPL / 4; d++) qw[d] = 0u;
    }
    return st;
}

// The lane's code sum (exact).
template <int VPL>
NQ_HD int q81_sum(const uint32_t (&qw)[VPL / 4]) {
    int sum = 0;
#pragma unroll
    for (int d = 0; d < VPL / 4; d++) sum = dot4(qw[d], 0x01010101u, sum);
    return sum;
}

// Phase 3 (after the code sums are combined): lane j of block b stores its
// codes; lane 0 stores the d and sum words.  Returns the block's status bits
// (lane 0 reports them).
template <int VPL>
NQ_HD uint32_t q81_store(const Q81Args &a, uint32_t b, uint32_t j, const uint32_t (&qw)[VPL / 4], uint32_t d16,
                         int sum, uint32_t st) {
    const uint32_t s16 = gq_f32_to_f16(f16(d16) * (float)sum);  // exact product, one rounding
    if ((s16 & 0x7C00u) == 0x7C00u) st |= 4u;
    uint32_t *blk = a.blocks + (uint64_t)b * 9u;
#pragma unroll
    for (int d = 0; d < VPL / 4; d++) blk[1u + j * (uint32_t)(VPL / 4) + (uint32_t)d] = qw[d];
    if (j == 0u) blk[0] = st & 3u ? 0u : d16 | s16 << 16;
    return st;
}

template <int IN, bool VECIN>
__global__ __launch_bounds__(WG) void k_quantize_q8_1(Q81Args a) {
    constexpr int VPL = gq_vpl<IN>();
    constexpr uint32_t LPB = q81_lanes<IN>();
    const uint32_t t = blockIdx.x * (uint32_t)WG + threadIdx.x;
    const uint32_t b = t / LPB, j = t % LPB;
    const bool live = b < a.nblocks;
    float v[VPL];
    uint32_t mag = 0u;
    if (live) {
        mag = gq_load<IN, VECIN>(GqDevSrc{a.x}, (uint64_t)b * 32u + j * (uint32_t)VPL, (uint32_t)VPL, v);
    } else {
#pragma unroll
        for (int k = 0; k < VPL; k++) v[k] = 0.0f;
    }
    // every lane of the wave takes part in the exchanges
#pragma unroll
    for (uint32_t off = LPB / 2; off >= 1; off >>= 1) mag = gq_umax(mag, (uint32_t)__shfl_xor((int)mag, (int)off, 64));
    uint32_t q[VPL / 4];
    uint32_t d16 = 0u;
    const uint32_t st = q81_encode<VPL>(mag, v, &d16, q);
    int sum = q81_sum<VPL>(q);
#pragma unroll
    for (uint32_t off = LPB / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, (int)off, 64);
    if (live) {
        const uint32_t bits = q81_store<VPL>(a, b, j, q, d16, sum, st);
        if (bits && j == 0u) atomicOr(a.status, bits);
    }
}

// ------------------------------------------------------------------ product

// Persistent waves: wave w of workgroup b takes rows 4b + w, 4b + w + step,
// ... (step = 4 * grid), so the grid sweeps the weight matrix front to back.
// A wave walks its rows in chunks of whole blocks (at most gv_chunk_bytes,
// 64 * gv_nl 16-byte groups at any start offset; two whole rows per chunk
// when they fit): while the lanes compute the current chunk from the wave's
// LDS region, the next chunk's loads (gv_nl coalesced 16-byte loads per
// lane) are already in flight.  The activation
// (codes, scales and exact code sums per 32-value block) is staged in LDS
// once per workgroup when it fits, so the compute phase touches LDS only and
// never waits on the prefetch.
// Per chunk a lane issues gv_nl<RW>() 16-byte loads: 5 when a chunk holds
// two or four rows (a pair of 2304-byte q4_k rows of 4096 values fits), else
// 4 (the measured best for single rows).
template <int RW>
constexpr int gv_nl() {
    return RW >= 2 ? 5 : 4;
}
// Chunk bytes: whole blocks spanning at most 64 * gv_nl 16-byte groups at any start offset.
template <int RW>
constexpr uint32_t gv_chunk_bytes() {
    return 1024u * (uint32_t)gv_nl<RW>() - 16u;
}
// LDS dwords per wave: the groups plus one group of padding.
template <int RW>
constexpr uint32_t gv_wave_dw() {
    return 4u * (64u * (uint32_t)gv_nl<RW>() + 1u);
}
constexpr uint32_t GV_WAVES = (uint32_t)WG / 64u;
constexpr uint32_t GV_ACT_LDS_MAX = 20480;                 // activation bytes staged in LDS at most

struct GvArgs {
    const uint32_t *wbase;  // weight bytes of this launch's first row, aligned down to 4 bytes
    uint32_t wmis;          // that row's start - wbase (0..3)
    uint32_t wlast;         // last dword holding weight bytes of this launch, from wbase
    const uint32_t *xq;     // q8_1 activation blocks; activation row m starts at dword m * xrow
    float *y;               // output of this launch's first weight row; activation row m at m * ldy
    uint32_t rows;          // weight rows in this launch
    uint32_t row_bytes;     // bytes per weight row, K / B * S
    uint32_t K;             // values per row
    uint32_t kb;            // activation blocks per row, K / 32
    uint32_t xrow;          // dwords per activation row, K / 32 * 9
    uint32_t ldy;           // N
    uint32_t M;             // activation rows, 1 .. MT
    uint32_t nbr;           // blocks per row
    uint32_t cb;            // blocks per chunk
    uint32_t rw;            // rows a chunk holds: 4 or 2 when that many whole rows fit one chunk, else 1
};

// Sum over the 64 lanes of a wave with DPP steps, in a fixed order: lane
// pairs, quads, half-rows and rows (each lane then holds its row's sum), then
// row 1 += row 0 and row 3 += row 2, then rows 2 and 3 += lane 31.  Lane 63
// holds ((r3 + r2) + (r1 + r0)), bit for bit the value of an XOR butterfly
// over offsets 1, 2, ..., 32 (every step adds two equal-shaped partials, and
// binary32 addition commutes).
template <int CTRL, int ROWS>
__device__ inline float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false);
    return v + __builtin_bit_cast(float, t);
}

__device__ inline float wave_sum63(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


constexpr uint32_t ONES8 = 0x01010101u;

// LDS dwords of the staged activation: M*K code bytes, then M*K/32 scales
// (binary32), then M*K/32 code sums (int32).
NQ_HD uint32_t gv_act_dw(const GvArgs &a) { return a.M * (a.K / 4u + 2u * a.kb); }

// Position of 16-byte code group g of an activation row in LDS: when K is a
// multiple of 128, group g sits at g ^ ((g >> 3) & 7) (a swap inside each
// aligned run of eight groups), so that lanes reading the groups of
// consecutive 32-value blocks (or of every other one) fall in distinct LDS
// banks; otherwise at g.
NQ_HD uint32_t act_group(uint32_t K, uint32_t g) { return (K & 127u) == 0u ? g ^ ((g >> 3) & 7u) : g; }

// Activation staging, strided over the workgroup's threads.
NQ_HD void gv_stage_act(const GvArgs &a, uint32_t *lds, uint32_t tid, uint32_t nthreads) {
    float *dl = (float *)(lds + a.M * a.K / 4u);
    int *sl = (int *)(dl + a.M * a.kb);
    for (uint32_t i = tid; i < a.M * a.kb; i += nthreads) {
        const uint32_t m = i / a.kb, blk = i - m * a.kb;
        const uint32_t *p = a.xq + (uint64_t)m * a.xrow + (uint64_t)blk * 9u;
        int sum = 0;
        uint32_t *row = lds + m * a.K / 4u;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t w = p[1 + j];
            row[4u * act_group(a.K, 2u * blk + (uint32_t)(j >> 2)) + (uint32_t)(j & 3)] = w;
            sum = dot4(ONES8, w, sum);
        }
        dl[i] = f16(p[0] & 0xFFFFu);
        sl[i] = sum;
    }
}

// Activation reader: q8_1 block ab of activation row m as its 8 code dwords,
// its scale (binary32) and the exact sum of its codes; from LDS, or from the
// blocks in global memory (the sum then computed).
template <bool ALDS>
struct GvAct {
    const uint32_t *xq;
    const uint32_t *lds;
    uint32_t K, kb, xrow, M;
    NQ_HD float block(uint32_t m, uint32_t ab, uint32_t (&c)[8], int *S) const {
        if constexpr (ALDS) {
            const uint32_t *row = lds + m * K / 4u;
            const uint32_t *c0 = row + 4u * act_group(K, 2u * ab), *c1 = row + 4u * act_group(K, 2u * ab + 1u);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                c[j] = c0[j];
                c[4 + j] = c1[j];
            }
            const float *dl = (const float *)(lds + M * K / 4u);
            *S = ((const int *)(dl + M * kb))[m * kb + ab];
            return dl[m * kb + ab];
        } else {
            const uint32_t *p = xq + (uint64_t)m * xrow + (uint64_t)ab * 9u;
            const u32x4a4 v0 = *(const u32x4a4 *)(p + 1), v1 = *(const u32x4a4 *)(p + 5);
            c[0] = v0.x; c[1] = v0.y; c[2] = v0.z; c[3] = v0.w;
            c[4] = v1.x; c[5] = v1.y; c[6] = v1.z; c[7] = v1.w;
            int s = 0;
#pragma unroll
            for (int j = 0; j < 8; j++) s = dot4(ONES8, c[j], s);
            *S = s;
            return f16(p[0] & 0xFFFFu);
        }
    }
};

// Items of the integer paths: a lane takes a group of weights of one block,
// decodes them to 8-bit integers and multiplies them with the activation
// codes of the same columns by 4-way dot products (exact integer sums); each
// exact sum is then scaled in binary32 and added to the lane's partial.
// Every gguf format has such a path.  An item is taken in three steps: its weights (gv_w, once per row), its
// activation columns (gv_a, once per activation row, shared by the rows of
// a chunk) and the product (gv_dot).
template <int F>
struct GvItem {
    // 32-value blocks (one item each)
    static constexpr bool B32 = F == Q4_0 || F == Q4_1 || F == Q5_0 || F == Q5_1 || F == Q8_0 || F == Q8_1 ||
                                F == IQ4_NL || F == MXFP4;
    // 256-value blocks in 32-value items (the IQ formats' 32-value groups)
    static constexpr bool IQ = F == IQ2_XXS || F == IQ2_XS || F == IQ2_S || F == IQ3_XXS || F == IQ3_S ||
                               F == IQ1_S || F == IQ1_M;
    static constexpr bool I32 = F == IQ4_XS || F == Q8_K || F == TQ2_0 || F == TQ1_0 || F == Q2_K || F == Q3_K || IQ;
    // 128- and 64-value blocks in 32-value items
    static constexpr bool S32 = F == Q1_0 || F == Q2_0;
    static constexpr bool INT = B32 || I32 || S32 || F == Q4_K || F == Q5_K || F == Q6_K || F == NVFP4_GGUF;
    static_assert(INT || F == NVFP4_DIV, "every gguf format takes integer items");
    // items per block
    static constexpr uint32_t IPB = B32 ? 1u : I32 ? 8u : S32 ? (uint32_t)block_values(F) / 32u
                                  : (F == Q4_K || F == Q5_K || F == Q6_K) ? 4u : 2u;
};

// 5-bit codes: byte k of the result is bit 4 of 16 * (bit k of b), k < 4
// (b's four low bits spread one per byte by a multiply that keeps the four
// shifted copies apart).
NQ_HD uint32_t spread4(uint32_t b) { return ((b & 15u) * 0x00204081u & 0x01010101u) << 4; }

// Four bits of b as four bytes 0 or 1 (the spread4 multiply without the shift).
NQ_HD uint32_t bits4(uint32_t b) { return (b & 15u) * 0x00204081u & 0x01010101u; }

// Byte mask of four sign bits: byte k is 0xFF when bit k of b is set.
NQ_HD uint32_t signmask4(uint32_t b) { return bits4(b) * 0xFFu; }

// The four 2-bit fields of byte b as four bytes (LSB field first).
NQ_HD uint32_t crumbs4(uint32_t b) { return (b | (b << 6) | (b << 12) | (b << 18)) & 0x03030303u; }

// IQ sign byte: seven stored bits and their parity as bit 7.
NQ_HD uint32_t iq_signs8(uint32_t s7) { return s7 | (parity7(s7) << 7); }

// Byte-wise c - o for bytes c < 128 and 0 <= o <= 128: no borrow crosses a
// byte, and the result bytes are the two's-complement differences.
NQ_HD uint32_t bsub(uint32_t c, uint32_t o) { return ((c | 0x80808080u) - o) ^ 0x80808080u; }


// The 32 base-3 digits (0..2, value order; the weight is digit - 1) of
// 32-value item p (< 8) of a tq1_0 block: values 32k + i (k < 5, i < 32)
// are digit k of byte i, values 160 + 16k + i (k < 5, i < 16) digit k of
// byte 32 + i, values 240 + 4k + i (k < 4, i < 4) digit k of byte 48 + i.
// Branch-free over the item (a wave's lanes take different items): each
// half reads one 16-byte window and takes one digit per byte, with the
// multiplier 3^k worked out once per half.
template <class Src>
NQ_HD void tq1_item(const Src &s, uint32_t bo, uint32_t p, uint32_t (&c)[8]) {
    const bool lo = p < 5u, tail = p == 7u;
    const uint32_t k1 = lo ? p : tail ? 4u : 2u * (p - 5u);
    const uint32_t m1 = pow3(k1), m2 = pow3(lo ? p : k1 + 1u);
    uint32_t q1[4], q2[4], h[1];
    window<4>(s, bo + (lo ? 0u : 32u), q1);
    window<4>(s, bo + (lo ? 16u : 32u), q2);
    window<1>(s, bo + 48u, h);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        c[j] = digits4m(q1[j], m1);
        c[4 + j] = digits4m(tail ? h[0] : q2[j], tail ? pow3((uint32_t)j) : m2);
    }
}

// Decoded weights of one item (the fields a format uses).
struct GvW {
    uint32_t q[16];
    float f[8];
};

// Activation columns of one item for one activation row: up to two q8_1
// blocks' codes, scales and exact code sums.
struct GvA {
    uint32_t c[16];
    float d[2];
    int S[2];
};

// The K-quant 6-bit sub-scale and min of sub-block k (0..7) from the 12
// packed bytes (three dwords), without branches: with j = k mod 4 and b1,
// b2, b3 byte j of the three dwords, k < 4 takes (b1 & 63, b2 & 63) and
// k >= 4 takes ((b3 & 15) | (b1 >> 6) << 4, (b3 >> 4) | (b2 >> 6) << 4).
NQ_HD void kq_scale_min(const uint32_t (&h)[3], uint32_t k, uint32_t *sc, uint32_t *mn) {
    const uint32_t sh = 8u * (k & 3u);
    const uint32_t b1 = (h[0] >> sh) & 0xFFu, b2 = (h[1] >> sh) & 0xFFu, b3 = (h[2] >> sh) & 0xFFu;
    const uint32_t hi = 0u - (uint32_t)(k >= 4u);  // all ones for k >= 4
    *sc = (((b3 & 15u) | ((b1 >> 6) << 4)) & hi) | ((b1 & 63u) & ~hi);
    *mn = (((b3 >> 4) | ((b2 >> 6) << 4)) & hi) | ((b2 & 63u) & ~hi);
}

// The sub-scales and mins of the pair of sub-blocks 2g, 2g + 1 (g < 4), as
// the bytes [sc(2g), sc(2g+1), m(2g), m(2g+1)] of one word, by byte selects:
// with j = 2g mod 4, A = [b1[j], b1[j+1], b2[j], b2[j+1]] gives the pair for
// g < 2 (6 low bits); for g >= 2 the low 4 bits come from b3[j], b3[j+1]
// (low nibbles for the scales, high for the mins) and bits 4-5 are bits 6-7
// of A's bytes.  Same values as kq_scale_min for k = 2g and 2g + 1.
NQ_HD uint32_t kq_scale_min_pair(const uint32_t (&h)[3], uint32_t g) {
    const uint32_t j = (2u * g) & 3u;
    const uint32_t sa = 0x05040100u + j * 0x01010101u;
    const uint32_t A = perm(h[1], h[0], sa);
    const uint32_t B = perm(h[2], h[2], sa - 0x04040000u);
    const uint32_t hi = (B & 0x00000F0Fu) | ((B >> 4) & 0x0F0F0000u) | ((A >> 2) & 0x30303030u);
    return g < 2u ? A & 0x3F3F3F3Fu : hi;
}

// A single-round wave region whose weight windows start at multiples of AL
// bytes (4 or 16): the launch's weight bytes start 16-byte aligned and, for
// the formats of gv_dword_windows, every block and every window the weight
// reader takes in it sits at a multiple of 4 bytes (of 16 for q4_k and q5_k,
// whose blocks are multiples of 16 bytes).  Windows are then plain dword
// loads (16-byte loads for AL = 16) with no byte shifts.
template <int AL>
struct LdsSrcAl : LdsSrc {};

template <int F>
constexpr int gv_dword_windows() {
    return (F == Q4_K || F == Q5_K) ? 16
         : (F == Q8_1 || F == Q8_K || F == Q4_1 || F == Q5_1 || F == IQ4_XS || F == NVFP4_GGUF || F == Q2_K) ? 4
                                                                                                         : 0;
}

template <class Src>
struct GvSrcAl {
    static constexpr int value = 0;
};
template <int AL>
struct GvSrcAl<LdsSrcAl<AL>> {
    static constexpr int value = AL;
};

// The single-round kernel's view of a wave region of format F.
template <int F>
using Gv1Src = std::conditional_t<(gv_dword_windows<F>() > 0), LdsSrcAl<gv_dword_windows<F>()>, LdsSrc>;

template <class Src>
NQ_HD Src gv_src(const uint32_t *base, uint32_t last) {
    Src s;
    s.base = base;
    s.last = last;
    return s;
}

// ND payload dwords from byte off of the source: window(), or plain loads
// from an aligned region.
template <int ND, class Src>
NQ_HD void gw_window(const Src &s, uint32_t off, uint32_t (&w)[ND]) {
    constexpr int AL = GvSrcAl<Src>::value;
    if constexpr (AL > 0) {
        const uint32_t *p = s.base + (off >> 2);
#if !defined(__HIP_DEVICE_COMPILE__)
        if (((uintptr_t)p & (uintptr_t)(AL - 1)) != 0u || (off & 3u) != 0u) __builtin_trap();
#endif
        if constexpr (AL == 16 && ND % 4 == 0) {
            const u32x4 *q = (const u32x4 *)__builtin_assume_aligned(p, 16);
#pragma unroll
            for (int k = 0; k < ND / 4; k++) {
                const u32x4 v = q[k];
                w[4 * k] = v.x;
                w[4 * k + 1] = v.y;
                w[4 * k + 2] = v.z;
                w[4 * k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < ND; k++) w[k] = p[k];
        }
    } else {
        window<ND>(s, off, w);
    }
}

// Weights of item `part` of the block at LDS byte offset bo.
template <int F, class Src>
NQ_HD void gv_w(const Src &s, uint32_t bo, uint32_t part, const Tab &tab, GvW &w) {
    if constexpr (F == Q8_0) {
        // d at 0, 32 signed codes at 2: w = d * q
        w.f[0] = f16(u16_at(s, bo));
        uint32_t q[8];
        gw_window<8>(s, bo + 2u, q);
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = q[j];
    } else if constexpr (F == Q4_0) {
        // d at 0, 16 bytes at 2: value j < 16 the low nibble of byte j, j >= 16
        // the high nibble of byte j - 16; w = d * (v - 8).  The nibbles are
        // split here, once per item (words 0-3 low, 4-7 high), not per
        // activation row.
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        w.f[0] = f16(u16_at(s, bo));
        uint32_t q[4];
        gw_window<4>(s, bo + 2u, q);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            w.q[j] = q[j] & LO4;
            w.q[4 + j] = (q[j] >> 4) & LO4;
        }
    } else if constexpr (F == Q8_1) {
        // d at 0, the sum at 2 (not used), 32 signed codes at 4: w = d * q
        w.f[0] = f16(u16_at(s, bo));
        uint32_t q[8];
        gw_window<8>(s, bo + 4u, q);
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = q[j];
    } else if constexpr (F == Q8_K) {
        // binary32 d at 0, 256 signed codes at 4 (part p: codes 32p .. 32p+31): w = RN32(d * q)
        uint32_t h[1], q[8];
        gw_window<1>(s, bo, h);
        gw_window<8>(s, bo + 4u + 32u * part, q);
        w.f[0] = bits_f32(h[0]);
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = q[j];
    } else if constexpr (F == Q4_1 || F == IQ4_NL || F == MXFP4) {
        // nibbles (value j < 16 the low nibble of byte j, j >= 16 the high
        // nibble of byte j - 16) of 16 bytes; q4_1: d at 0, m at 2, bytes at
        // 4, w = d * v + m; iq4_nl: d at 0, bytes at 2, w = d * IQ4[v];
        // mxfp4: E8M0 byte at 0, bytes at 1, w = half-scale * V[v] (the
        // doubled E2M1 table)
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        uint32_t q[4];
        if constexpr (F == Q4_1) {
            w.f[0] = f16(u16_at(s, bo));
            w.f[1] = f16(u16_at(s, bo + 2u));
            gw_window<4>(s, bo + 4u, q);
        } else if constexpr (F == IQ4_NL) {
            w.f[0] = f16(u16_at(s, bo));
            gw_window<4>(s, bo + 2u, q);
        } else {
            const uint32_t e = u8_at(s, bo);
            w.f[0] = bits_f32(e < 2u ? (0x00200000u << e) : ((e - 1u) << 23));
            gw_window<4>(s, bo + 1u, q);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t lo = q[j] & LO4, hi = (q[j] >> 4) & LO4;
            if constexpr (F == Q4_1) {
                w.q[j] = lo;
                w.q[4 + j] = hi;
            } else if constexpr (F == IQ4_NL) {
                w.q[j] = lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, lo);
                w.q[4 + j] = lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, hi);
            } else {
                w.q[j] = lut16(FP4T0, FP4T1, FP4T2, FP4T3, lo);
                w.q[4 + j] = lut16(FP4T0, FP4T1, FP4T2, FP4T3, hi);
            }
        }
    } else if constexpr (F == Q5_0 || F == Q5_1) {
        // value j = nibble j (as q4_0) + 16 * bit j of the 32-bit high word;
        // q5_0: d at 0, high at 2, bytes at 6, w = d * (v - 16); q5_1: d at 0,
        // m at 2, high at 4, bytes at 8, w = d * v + m
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        const uint32_t ho = F == Q5_0 ? 2u : 4u;
        uint32_t hw[1], q[4];
        gw_window<1>(s, bo + ho, hw);
        gw_window<4>(s, bo + ho + 4u, q);
        w.f[0] = f16(u16_at(s, bo));
        if constexpr (F == Q5_1) w.f[1] = f16(u16_at(s, bo + 2u));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            w.q[j] = (q[j] & LO4) | spread4(hw[0] >> (4 * j));
            w.q[4 + j] = ((q[j] >> 4) & LO4) | spread4(hw[0] >> (16 + 4 * j));
        }
    } else if constexpr (F == IQ4_XS) {
        // part k: values 32k .. 32k+31, nibbles (as q4_0) of bytes 8 + 16k ..;
        // w = RN32(d * s_k) * IQ4[v], s_k = scale nibble k + 16 * high bits 2k,2k+1 - 32
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        uint32_t hdr[2], q[4];
        gw_window<2>(s, bo, hdr);
        gw_window<4>(s, bo + 8u + 16u * part, q);
        const float d = f16(hdr[0] & 0xFFFFu);
        const uint32_t high = hdr[0] >> 16;
        const uint32_t lo = (bytek(hdr[1], part >> 1) >> (4u * (part & 1u))) & 15u;
        const uint32_t sk = lo + 16u * ((high >> (2u * part)) & 3u);
        w.f[0] = M(d, (float)((int)sk - 32));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            w.q[j] = lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, q[j] & LO4);
            w.q[4 + j] = lut16(IQ4T0, IQ4T1, IQ4T2, IQ4T3, (q[j] >> 4) & LO4);
        }
    } else if constexpr (F == TQ2_0) {
        // part c: values 32c + i, bits 2(c mod 4) of byte 32(c / 4) + i; d at
        // 64; w = d * (v - 1)
        uint32_t q[8];
        gw_window<8>(s, bo + 32u * (part >> 2), q);
        w.f[0] = f16(u16_at(s, bo + 64u));
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = (q[j] >> (2u * (part & 3u))) & 0x03030303u;
    } else if constexpr (F == TQ1_0) {
        // part p: 32 base-3 digits v (tq1_item); d at 52; w = d * (v - 1)
        uint32_t c[8];
        tq1_item(s, bo, part, c);
        w.f[0] = f16(u16_at(s, bo + 52u));
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = c[j];
    } else if constexpr (F == NVFP4_GGUF) {
        // part p: groups 2p and 2p+1 (16 values each); group g's E4M3 scale
        // byte at g, its codes the low then the high nibbles of bytes
        // 4 + 8g .. 4 + 8g + 7; w = half-scale(g) * V[v]
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        uint32_t q[4];
        gw_window<4>(s, bo + 4u + 16u * part, q);
        const uint32_t sb = u16_at(s, bo + 2u * part);
        w.f[0] = nvfp4_half_scale(sb & 0xFFu);
        w.f[1] = nvfp4_half_scale(sb >> 8);
#pragma unroll
        for (int e = 0; e < 2; e++) {
            w.q[4 * e + 0] = lut16(FP4T0, FP4T1, FP4T2, FP4T3, q[2 * e] & LO4);
            w.q[4 * e + 1] = lut16(FP4T0, FP4T1, FP4T2, FP4T3, q[2 * e + 1] & LO4);
            w.q[4 * e + 2] = lut16(FP4T0, FP4T1, FP4T2, FP4T3, (q[2 * e] >> 4) & LO4);
            w.q[4 * e + 3] = lut16(FP4T0, FP4T1, FP4T2, FP4T3, (q[2 * e + 1] >> 4) & LO4);
        }
    } else if constexpr (F == Q5_K) {
        // part g as q4_k, codes from bytes 48 + 32g .. plus 16 * bit 2g (low
        // half) or 2g+1 (high half) of bytes 16 .. 47
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        uint32_t h[4], q[8], qh[8];
        gw_window<4>(s, bo, h);
        gw_window<8>(s, bo + 48u + 32u * part, q);
        gw_window<8>(s, bo + 16u, qh);
        const float d = f16(h[0] & 0xFFFFu), dmin = f16(h[0] >> 16);
        const uint32_t hs[3] = {h[1], h[2], h[3]};
        const uint32_t sm = kq_scale_min_pair(hs, part);
        w.f[0] = M(d, (float)bytek(sm, 0u));
        w.f[1] = M(dmin, (float)bytek(sm, 2u));
        w.f[2] = M(d, (float)bytek(sm, 1u));
        w.f[3] = M(dmin, (float)bytek(sm, 3u));
#pragma unroll
        for (int j = 0; j < 8; j++) {
            w.q[j] = (q[j] & LO4) | (((qh[j] >> (2u * part)) & 0x01010101u) << 4);
            w.q[8 + j] = ((q[j] >> 4) & LO4) | (((qh[j] >> (2u * part + 1u)) & 0x01010101u) << 4);
        }
    } else if constexpr (F == Q2_K) {
        // part c: values 32c + i, bits 2(c mod 4) of byte 16 + 32(c / 4) + i;
        // sub-block scale bytes 2c, 2c+1 (low nibble: scale, high: min);
        // d at 80, dmin at 82; w = RN32(d * (s mod 16)) * v - RN32(dmin * (s / 16))
        uint32_t q[8], h[1];
        gw_window<8>(s, bo + 16u + 32u * (part >> 2), q);
        gw_window<1>(s, bo + 80u, h);
        const uint32_t sc = u16_at(s, bo + 2u * part);
        const float d = f16(h[0] & 0xFFFFu), dmin = f16(h[0] >> 16);
        w.f[0] = M(d, (float)(sc & 15u));
        w.f[1] = M(dmin, (float)((sc >> 4) & 15u));
        w.f[2] = M(d, (float)((sc >> 8) & 15u));
        w.f[3] = M(dmin, (float)(sc >> 12));
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = (q[j] >> (2u * (part & 3u))) & 0x03030303u;
    } else if constexpr (F == Q3_K) {
        // part c: v = bits 2(c mod 4) of byte 32 + 32(c / 4) + i, plus 4 * bit c
        // of mask byte i; code v + 4h - 4; sub-block k scale l + 16a - 32 (l:
        // nibble k / 8 of byte 96 + k mod 8, a: bits 2(k / 4) of byte 104 + k
        // mod 4); d at 108; w = RN32(d * s) * (v - 4 (1 - h))
        uint32_t q[8], mk[8], sc[3];
        gw_window<8>(s, bo + 32u + 32u * (part >> 2), q);
        gw_window<8>(s, bo, mk);
        gw_window<3>(s, bo + 96u, sc);
        const float d = f16(u16_at(s, bo + 108u));
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const uint32_t k = 2u * part + (uint32_t)e, lk = k & 7u;
            const uint32_t l = (bytek(lk < 4u ? sc[0] : sc[1], lk & 3u) >> (4u * (k >> 3))) & 15u;
            const uint32_t a = (bytek(sc[2], k & 3u) >> (2u * (k >> 2))) & 3u;
            w.f[e] = M(d, (float)((int)(l + 16u * a) - 32));
        }
#pragma unroll
        for (int j = 0; j < 8; j++)
            w.q[j] = ((q[j] >> (2u * (part & 3u))) & 0x03030303u) | (((mk[j] >> part) & 0x01010101u) << 2);
    } else if constexpr (F == Q1_0) {
        // part p: values 32p + i, bit i mod 8 of byte 2 + 4p + i / 8; w = +-d (d
        // for a set bit): code 2b - 1
        uint32_t q[1];
        gw_window<1>(s, bo + 2u + 4u * part, q);
        w.f[0] = f16(u16_at(s, bo));
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = bits4(q[0] >> (4 * j));
    } else if constexpr (F == Q2_0) {
        // part p: values 32p + 4t + k, bits 2k of byte 2 + 8p + t; w = d * (v - 1)
        uint32_t q[2];
        gw_window<2>(s, bo + 2u + 8u * part, q);
        w.f[0] = f16(u16_at(s, bo));
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = crumbs4(bytek(q[j >> 2], (uint32_t)(j & 3)));
    } else if constexpr (GvItem<F>::IQ) {
        // group g = part (32 values, units 4g .. 4g+3): per unit its 8 grid
        // bytes (w.q[2l], w.q[2l+1]) and those bytes under its negative signs
        // (w.q[8 + 2l], w.q[9 + 2l]); the scales in w.f (see gv_dot)
        const uint32_t g = part;
        const float d = F == IQ1_M ? 0.0f : f16(u16_at(s, bo));
        if constexpr (F == IQ2_XXS || F == IQ3_XXS) {
            // iq2_xxs: 4 index bytes then the aux word at 2 + 8g; iq3_xxs: index
            // pairs at 2 + 8g, the aux word at 66 + 4g; seven sign bits per unit
            // (+ parity), scale nibble aux >> 28
            uint32_t ix[2], aux[1];
            gw_window<2>(s, bo + 2u + 8u * g, ix);
            if constexpr (F == IQ2_XXS)
                aux[0] = ix[1];
            else
                gw_window<1>(s, bo + 66u + 4u * g, aux);
            w.f[0] = M(M(d, A(0.5f, (float)(aux[0] >> 28))), F == IQ2_XXS ? 0.25f : 0.5f);
#pragma unroll
            for (int l = 0; l < 4; l++) {
                uint32_t g0, g1;
                if constexpr (F == IQ2_XXS) {
                    const uint64_t row = tab.iq2xxs(bytek(ix[0], (uint32_t)l));
                    g0 = (uint32_t)row;
                    g1 = (uint32_t)(row >> 32);
                } else {
                    const uint32_t i2 = (ix[l >> 1] >> (16 * (l & 1))) & 0xFFFFu;
                    g0 = tab.iq3xxs(i2 & 0xFFu);
                    g1 = tab.iq3xxs(i2 >> 8);
                }
                const uint32_t sg = iq_signs8((aux[0] >> (7u * (uint32_t)l)) & 127u);
                w.q[2 * l] = g0;
                w.q[2 * l + 1] = g1;
                w.q[8 + 2 * l] = g0 & signmask4(sg);
                w.q[9 + 2 * l] = g1 & signmask4(sg >> 4);
            }
        } else if constexpr (F == IQ2_XS || F == IQ2_S) {
            // two scale nibbles per group (units 0-1 and 2-3): iq2_xs at byte
            // 66 + g, iq2_s at 74 + g; c = RN32(RN32(d * (0.5 + t)) * 0.25)
            const uint32_t sb = u8_at(s, bo + (F == IQ2_XS ? 66u : 74u) + g);
            w.f[0] = M(M(d, A(0.5f, (float)(sb & 15u))), 0.25f);
            w.f[1] = M(M(d, A(0.5f, (float)(sb >> 4))), 0.25f);
            uint32_t wd[2], lo[1], sgn[1];
            uint32_t hi = 0;
            if constexpr (F == IQ2_XS) {
                gw_window<2>(s, bo + 2u + 8u * g, wd);  // four 16-bit words: 9-bit index, 7 sign bits
            } else {
                gw_window<1>(s, bo + 2u + 4u * g, lo);   // four index low bytes
                gw_window<1>(s, bo + 34u + 4u * g, sgn); // four sign bytes
                hi = u8_at(s, bo + 66u + g);          // four 2-bit index high parts
            }
#pragma unroll
            for (int l = 0; l < 4; l++) {
                uint64_t row;
                uint32_t sg;
                if constexpr (F == IQ2_XS) {
                    const uint32_t word = (wd[l >> 1] >> (16 * (l & 1))) & 0xFFFFu;
                    row = tab.iq2xs(word & 511u);
                    sg = iq_signs8(word >> 9);
                } else {
                    row = tab.iq2s(bytek(lo[0], (uint32_t)l) | (((hi >> (2 * l)) & 3u) << 8));
                    sg = bytek(sgn[0], (uint32_t)l);
                }
                const uint32_t g0 = (uint32_t)row, g1 = (uint32_t)(row >> 32);
                w.q[2 * l] = g0;
                w.q[2 * l + 1] = g1;
                w.q[8 + 2 * l] = g0 & signmask4(sg);
                w.q[9 + 2 * l] = g1 & signmask4(sg >> 4);
            }
        } else if constexpr (F == IQ3_S) {
            // index pairs at 2 + 8g with a ninth bit each from byte 66 + g, sign
            // bytes at 74 + 4g, scale nibble g mod 2 of byte 106 + g / 2:
            // c = RN32(d * (1 + 2 t))
            uint32_t ix[2], sgn[1];
            gw_window<2>(s, bo + 2u + 8u * g, ix);
            gw_window<1>(s, bo + 74u + 4u * g, sgn);
            const uint32_t h = u8_at(s, bo + 66u + g);
            const uint32_t sc = u8_at(s, bo + 106u + (g >> 1));
            w.f[0] = M(d, (float)(1u + 2u * ((sc >> (4u * (g & 1u))) & 15u)));
#pragma unroll
            for (int l = 0; l < 4; l++) {
                const uint32_t i2 = (ix[l >> 1] >> (16 * (l & 1))) & 0xFFFFu;
                const uint32_t g0 = tab.iq3s((i2 & 0xFFu) | (((h >> (2 * l)) & 1u) << 8));
                const uint32_t g1 = tab.iq3s((i2 >> 8) | (((h >> (2 * l + 1)) & 1u) << 8));
                const uint32_t sg = bytek(sgn[0], (uint32_t)l);
                w.q[2 * l] = g0;
                w.q[2 * l + 1] = g1;
                w.q[8 + 2 * l] = g0 & signmask4(sg);
                w.q[9 + 2 * l] = g1 & signmask4(sg >> 4);
            }
        } else if constexpr (F == IQ1_S) {
            // index low bytes at 2 + 4g, the group word a at 34 + 2g (3 index
            // bits per unit, scale bits 12-14, delta sign bit 15); grid bytes
            // hold value + 1; w = RN32(d * (2 t + 1)) * (v + delta)
            uint32_t ix[1];
            gw_window<1>(s, bo + 2u + 4u * g, ix);
            const uint32_t a = u16_at(s, bo + 34u + 2u * g);
            w.f[0] = M(d, (float)(2u * ((a >> 12) & 7u) + 1u));
            w.f[1] = (a & 0x8000u) ? -0.125f : 0.125f;
#pragma unroll
            for (int l = 0; l < 4; l++) {
                const uint64_t row = tab.iq1s(bytek(ix[0], (uint32_t)l) | (((a >> (3 * l)) & 7u) << 8));
                w.q[2 * l] = (uint32_t)row;
                w.q[2 * l + 1] = (uint32_t)(row >> 32);
            }
        } else {  // IQ1_M
            // index low bytes at 4g, a nibble per unit (bytes 32 + 2g, 33 + 2g:
            // 3 index bits, delta sign bit 3), scale words at 48 (3 bits per
            // pair of units; the binary16 d in their top nibbles)
            uint32_t ix[1], hw[1], sw[2];
            gw_window<1>(s, bo + 4u * g, ix);
            gw_window<1>(s, bo + 32u + 2u * g, hw);  // the unit nibbles of this group (low 16 bits)
            gw_window<2>(s, bo + 48u, sw);
            const uint32_t dbits = ((sw[0] & 0xFFFFu) >> 12) | ((sw[0] >> 28) << 4) | (((sw[1] & 0xFFFFu) >> 12) << 8) |
                                   ((sw[1] >> 28) << 12);
            const float dm = f16(dbits);
            const uint32_t kw = g >> 1;
            const uint32_t wg = ((kw >> 1) == 0u ? sw[0] : sw[1]) >> (16u * (kw & 1u));
#pragma unroll
            for (int p = 0; p < 2; p++) {
                const uint32_t t = (wg >> (6u * (g & 1u) + 3u * (uint32_t)p)) & 7u;
                w.f[p] = M(dm, (float)(2u * t + 1u));
            }
#pragma unroll
            for (int l = 0; l < 4; l++) {
                const uint32_t an = (hw[0] >> (4 * l)) & 15u;
                const uint64_t row = tab.iq1s(bytek(ix[0], (uint32_t)l) | ((an & 7u) << 8));
                w.q[2 * l] = (uint32_t)row;
                w.q[2 * l + 1] = (uint32_t)(row >> 32);
                w.f[2 + l] = (an & 8u) ? -0.125f : 0.125f;
            }
        }
    } else if constexpr (F == Q4_K) {
        // part g: values 64g .. 64g+63, the low (sub-block 2g) and high
        // (sub-block 2g+1) nibbles of bytes 16 + 32g .. 16 + 32g + 31;
        // w = RN32(d * sc) * v - RN32(dmin * m)
        uint32_t h[4], q[8];
        gw_window<4>(s, bo, h);
        gw_window<8>(s, bo + 16u + 32u * part, q);
        const float d = f16(h[0] & 0xFFFFu), dmin = f16(h[0] >> 16);
        const uint32_t hs[3] = {h[1], h[2], h[3]};
        const uint32_t sm = kq_scale_min_pair(hs, part);
        w.f[0] = M(d, (float)bytek(sm, 0u));
        w.f[1] = M(dmin, (float)bytek(sm, 2u));
        w.f[2] = M(d, (float)bytek(sm, 1u));
        w.f[3] = M(dmin, (float)bytek(sm, 3u));
        // the code bytes as they are (gv_dot splits the nibbles: holding
        // both halves here took the two-row kernels with several activation
        // rows from 65 to 81 registers)
#pragma unroll
        for (int j = 0; j < 8; j++) w.q[j] = q[j];
    } else if constexpr (F == Q6_K) {
        // part p = 2h + c0: values 128h + 32c + i (i < 32) for c = c0 and
        // c0 + 2: low 4 bits from byte 64h + 32c0 + i (low nibble for c0,
        // high for c0 + 2), high 2 bits from byte 128 + 32h + i (bits 2c);
        // w = RN32(d * sc[16-value sub-block]) * (v - 32)
        constexpr uint32_t LO4 = 0x0F0F0F0Fu;
        const uint32_t hh = part >> 1, c0 = part & 1u;
        uint32_t ql[8], qh[8], sw[2];
        gw_window<8>(s, bo + 64u * hh + 32u * c0, ql);
        gw_window<8>(s, bo + 128u + 32u * hh, qh);
        gw_window<2>(s, bo + 192u + 8u * hh + 2u * c0, sw);
        const float d = f16(u16_at(s, bo + 208u));
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const uint32_t c = c0 + 2u * (uint32_t)e;
#pragma unroll
            for (int j = 0; j < 8; j++)
                w.q[8 * e + j] = ((e ? ql[j] >> 4 : ql[j]) & LO4) | (((qh[j] >> (2u * c)) & 0x03030303u) << 4);
            w.f[2 * e] = M(d, (float)(int8_t)(sw[e] & 0xFFu));
            w.f[2 * e + 1] = M(d, (float)(int8_t)((sw[e] >> 8) & 0xFFu));
        }
    } else {
        static_assert(F < 0, "format without integer items");
    }
}

// Activation columns of item `part` of block b (the block's index in its
// row) for activation row m.
template <int F, class Act>
NQ_HD void gv_a(const Act &act, uint32_t m, uint32_t b, uint32_t part, GvA &x) {
    uint32_t c[8];
    if constexpr (GvItem<F>::B32 || GvItem<F>::I32 || GvItem<F>::S32 || F == NVFP4_GGUF) {
        // the item's 32 values are activation block b (32-value blocks) or
        // IPB b + part (32-value items of larger blocks)
        const uint32_t ab = GvItem<F>::B32 ? b : GvItem<F>::IPB * b + part;
        x.d[0] = act.block(m, ab, c, &x.S[0]);
#pragma unroll
        for (int j = 0; j < 8; j++) x.c[j] = c[j];
    } else if constexpr (F == Q4_K || F == Q5_K || F == Q6_K) {
        // q4_k / q5_k: blocks 8b + 2g and 8b + 2g + 1; q6_k: 8b + 4h + c0 and 8b + 4h + c0 + 2
        const uint32_t ab = F != Q6_K ? 8u * b + 2u * part : 8u * b + 4u * (part >> 1) + (part & 1u);
        const uint32_t ab1 = F != Q6_K ? ab + 1u : ab + 2u;
        x.d[0] = act.block(m, ab, c, &x.S[0]);
#pragma unroll
        for (int j = 0; j < 8; j++) x.c[j] = c[j];
        x.d[1] = act.block(m, ab1, c, &x.S[1]);
#pragma unroll
        for (int j = 0; j < 8; j++) x.c[8 + j] = c[j];
    } else {
        static_assert(F < 0, "format without integer items");
    }
}

// The item's product with one activation row, added to acc.
template <int F>
NQ_HD float gv_dot(const GvW &w, const GvA &x, float acc) {
    constexpr uint32_t LO4 = 0x0F0F0F0Fu;
    if constexpr (F == Q8_0 || F == Q8_1 || F == Q8_K || F == IQ4_NL || F == MXFP4 || F == IQ4_XS) {
        // w = scale * (8-bit integer): the scale times the exact dot product
        int I = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) I = dot4(w.q[j], x.c[j], I);
        return __builtin_fmaf(w.f[0] * (float)I, x.d[0], acc);
    } else if constexpr (F == Q4_1 || F == Q5_1) {
        // w = d * v + m: d times the dot product plus m times the codes' sum
        int I = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) I = dot4(w.q[j], x.c[j], I);
        return __builtin_fmaf(w.f[0] * (float)I + w.f[1] * (float)x.S[0], x.d[0], acc);
    } else if constexpr (F == Q5_0 || F == TQ2_0 || F == TQ1_0) {
        // w = d * (v - o), o = 16 or 1: exact integer offset through the codes' sum
        constexpr int O = F == Q5_0 ? 16 : 1;
        int I = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) I = dot4(w.q[j], x.c[j], I);
        return __builtin_fmaf(w.f[0] * (float)(I - O * x.S[0]), x.d[0], acc);
    } else if constexpr (F == NVFP4_GGUF) {
        // two 16-value groups with their own scales in one activation block
        int I0 = 0, I1 = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            I0 = dot4(w.q[j], x.c[j], I0);
            I1 = dot4(w.q[4 + j], x.c[4 + j], I1);
        }
        return __builtin_fmaf(w.f[0] * (float)I0 + w.f[1] * (float)I1, x.d[0], acc);
    } else if constexpr (F == Q2_K) {
        // two 16-value sub-blocks, each RN32(d * s) * I - RN32(dmin * m) * S
        int I0 = 0, I1 = 0, S0 = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            I0 = dot4(w.q[j], x.c[j], I0);
            S0 = dot4(ONES8, x.c[j], S0);
            I1 = dot4(w.q[4 + j], x.c[4 + j], I1);
        }
        const int S1 = x.S[0] - S0;
        return __builtin_fmaf((w.f[0] * (float)I0 - w.f[1] * (float)S0) + (w.f[2] * (float)I1 - w.f[3] * (float)S1),
                              x.d[0], acc);
    } else if constexpr (F == Q3_K) {
        // two 16-value sub-blocks of codes v + 4h - 4
        int I0 = 0, I1 = 0, S0 = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            I0 = dot4(w.q[j], x.c[j], I0);
            S0 = dot4(ONES8, x.c[j], S0);
            I1 = dot4(w.q[4 + j], x.c[4 + j], I1);
        }
        const int S1 = x.S[0] - S0;
        return __builtin_fmaf(w.f[0] * (float)(I0 - 4 * S0) + w.f[1] * (float)(I1 - 4 * S1), x.d[0], acc);
    } else if constexpr (F == Q1_0 || F == Q2_0) {
        // q1_0: codes 2b - 1; q2_0: v - 1
        int I = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) I = dot4(w.q[j], x.c[j], I);
        const int V = F == Q1_0 ? 2 * I - x.S[0] : I - x.S[0];
        return __builtin_fmaf(w.f[0] * (float)V, x.d[0], acc);
    } else if constexpr (F == IQ2_XXS || F == IQ3_XXS || F == IQ3_S) {
        // signed grid values: dot(g, x) - 2 dot(g under the negative signs, x); one scale
        int I = 0, N = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            I = dot4(w.q[j], x.c[j], I);
            N = dot4(w.q[8 + j], x.c[j], N);
        }
        return __builtin_fmaf(w.f[0] * (float)(I - 2 * N), x.d[0], acc);
    } else if constexpr (F == IQ2_XS || F == IQ2_S) {
        // as above with a scale per pair of units (words 0-3: units 0-1)
        int I0 = 0, I1 = 0, N0 = 0, N1 = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            I0 = dot4(w.q[j], x.c[j], I0);
            N0 = dot4(w.q[8 + j], x.c[j], N0);
            I1 = dot4(w.q[4 + j], x.c[4 + j], I1);
            N1 = dot4(w.q[12 + j], x.c[4 + j], N1);
        }
        return __builtin_fmaf(w.f[0] * (float)(I0 - 2 * N0) + w.f[1] * (float)(I1 - 2 * N1), x.d[0], acc);
    } else if constexpr (F == IQ1_S) {
        // codes are grid bytes - 1: dot(g, x) - S; plus delta * S; one scale
        int I = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) I = dot4(w.q[j], x.c[j], I);
        const float T = (float)(I - x.S[0]) + w.f[1] * (float)x.S[0];  // exact: integers and eighths
        return __builtin_fmaf(w.f[0] * T, x.d[0], acc);
    } else if constexpr (F == IQ1_M) {
        // per unit: dot(g, x) - S_l + delta_l * S_l (S_l the unit's 8 codes);
        // a scale per pair of units
        float T[2] = {0.0f, 0.0f};
#pragma unroll
        for (int l = 0; l < 4; l++) {
            const int Sl = dot4(ONES8, x.c[2 * l + 1], dot4(ONES8, x.c[2 * l], 0));
            const int Il = dot4(w.q[2 * l + 1], x.c[2 * l + 1], dot4(w.q[2 * l], x.c[2 * l], 0));
            T[l >> 1] = T[l >> 1] + ((float)(Il - Sl) + w.f[2 + l] * (float)Sl);  // exact: integers and eighths
        }
        return __builtin_fmaf(w.f[0] * T[0] + w.f[1] * T[1], x.d[0], acc);
    } else if constexpr (F == Q4_0) {
        int I = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            I = dot4(w.q[j], x.c[j], I);
            I = dot4(w.q[4 + j], x.c[4 + j], I);
        }
        return __builtin_fmaf(w.f[0] * (float)(I - 8 * x.S[0]), x.d[0], acc);
    } else if constexpr (F == Q4_K || F == Q5_K) {
        int I0 = 0, I1 = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            if constexpr (F == Q4_K) {
                // high nibbles as the signed bytes (q & 0xF0) ^ 0x80 = 16 v - 128
                // (one 3-input bitwise instruction): the dot product D with
                // the second block's codes is 16 I1 - 128 S1, S1 their sum
                I0 = dot4(w.q[j] & LO4, x.c[j], I0);
                I1 = dot4((w.q[j] & 0xF0F0F0F0u) ^ 0x80808080u, x.c[8 + j], I1);
            } else {
                I0 = dot4(w.q[j], x.c[j], I0);
                I1 = dot4(w.q[8 + j], x.c[8 + j], I1);
            }
        }
        if constexpr (F == Q4_K) I1 = (I1 + x.S[1] * 128) >> 4;  // exact: D + 128 S1 = 16 I1
        acc = __builtin_fmaf(w.f[0] * (float)I0 - w.f[1] * (float)x.S[0], x.d[0], acc);
        return __builtin_fmaf(w.f[2] * (float)I1 - w.f[3] * (float)x.S[1], x.d[1], acc);
    } else if constexpr (F == Q6_K) {
#pragma unroll
        for (int e = 0; e < 2; e++) {
            int I0 = 0, I1 = 0, S0 = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                I0 = dot4(w.q[8 * e + j], x.c[8 * e + j], I0);
                S0 = dot4(ONES8, x.c[8 * e + j], S0);
                I1 = dot4(w.q[8 * e + 4 + j], x.c[8 * e + 4 + j], I1);
            }
            const int S1 = x.S[e] - S0;
            acc = __builtin_fmaf(w.f[2 * e] * (float)(I0 - 32 * S0) + w.f[2 * e + 1] * (float)(I1 - 32 * S1),
                                 x.d[e], acc);
        }
        return acc;
    } else {
        static_assert(F < 0, "format without integer items");
        return acc;
    }
}

// A chunk: blocks c0 .. c0+nb-1 of rows r .. r+rw-1 (rw > 1 only for whole
// rows), spanning 16-byte groups g0..g1 of the launch's weight bytes; its
// first block sits at LDS byte o0 of the wave's region, row r+i's at
// o0 + i * row_bytes.
struct GvChunk {
    uint32_t r, rw, c0, nb, g0, g1, o0;
};

NQ_HD GvChunk gv_chunk(const GvArgs &a, uint32_t r, uint32_t c0) {
    const uint32_t S = a.row_bytes / a.nbr;
    GvChunk c;
    c.r = r;
    c.rw = a.rows - r < a.rw ? a.rows - r : a.rw;
    c.c0 = c0;
    c.nb = a.nbr - c0 < a.cb ? a.nbr - c0 : a.cb;
    const uint32_t p0 = a.wmis + r * a.row_bytes + c0 * S;
    const uint32_t p1 = p0 + (c.rw - 1u) * a.row_bytes + c.nb * S - 1u;
    c.g0 = p0 >> 4;
    c.g1 = p1 >> 4;
    c.o0 = p0 & 15u;
    return c;
}

// The chunk after (r, c0) in a wave's sequence: the row's next chunk, else
// the first chunk of the wave's next row group (step groups of rw rows on).
NQ_HD void gv_advance(const GvArgs &a, uint32_t step, uint32_t *r, uint32_t *c0) {
    *c0 += a.cb;
    if (*c0 >= a.nbr) {
        *c0 = 0u;
        *r += step * a.rw;
    }
}

// Chunk staging, lane part, in two steps: the lane's NL 16-byte loads
// of groups g0 + lane + 64k (clamped to g1: lanes past the chunk repeat its
// last group, same address and value) into registers, and later their
// stores into the wave's LDS region (group g at dword 4 (g - g0)).  A group
// that passes the last weight dword (wlast) is loaded as the 16 bytes that
// end there and shifted into place, zero-filled; every load is in bounds
// (a launch holds at least 16 bytes) and none depends on a branch.
template <int NL, class Src>
NQ_HD void gv_issue(const Src &src, uint32_t wlast, const GvChunk &c, uint32_t lane, uint32_t (&v)[NL][4]) {
#pragma unroll
    for (int k = 0; k < NL; k++) {
        const uint32_t g0 = c.g0 + lane + 64u * (uint32_t)k;
        const uint32_t i = 4u * (g0 < c.g1 ? g0 : c.g1);
        src.load_stream4(i + 3u <= wlast ? i : wlast - 3u, v[k]);
    }
}

// The stores of gv_issue's loads (the shift of a group that passed wlast is
// applied here, once the data has arrived, so the loads stay in flight
// until then).
template <int NL>
NQ_HD void gv_put(const GvChunk &c, uint32_t wlast, uint32_t lane, const uint32_t (&v)[NL][4], uint32_t *lds) {
    const bool whole = 4u * c.g1 + 3u <= wlast;  // the same for the whole wave: only a launch's last group passes
#pragma unroll
    for (int k = 0; k < NL; k++) {
        const uint32_t g0 = c.g0 + lane + 64u * (uint32_t)k, g = g0 < c.g1 ? g0 : c.g1;
        uint32_t *d = lds + 4u * (g - c.g0);
        if (whole) {
            d[0] = v[k][0];
            d[1] = v[k][1];
            d[2] = v[k][2];
            d[3] = v[k][3];
        } else {
            const uint32_t i = 4u * g, sh = i + 3u <= wlast ? 0u : i - (wlast - 3u);  // 0 .. 3
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t x1 = e + 1 < 4 ? v[k][e + 1] : 0u, x2 = e + 2 < 4 ? v[k][e + 2] : 0u,
                               x3 = e + 3 < 4 ? v[k][e + 3] : 0u;
                d[e] = sh == 0u ? v[k][e] : sh == 1u ? x1 : sh == 2u ? x2 : x3;
            }
        }
    }
}

// A lane's positions of a staged chunk (items lane, lane + 64, ... of one
// row's blocks c0..c0+nb-1): per position the weights of each of the chunk's
// rows, then per activation row its columns, used by every row.
template <int F, int MT, int RW, class Act, class Src>
NQ_HD void gv_chunk_items(const Src &s, const GvChunk &c, uint32_t lane, uint32_t nm, uint32_t row_bytes,
                          const Act &act, const Tab &tab, float (&acc)[RW][MT]) {
    constexpr uint32_t IPB = GvItem<F>::IPB, S = (uint32_t)block_bytes(F);
    const uint32_t n = c.nb * IPB;
    for (uint32_t i = lane; i < n; i += 64u) {
        const uint32_t bl = i / IPB, part = i - bl * IPB;
        GvW w[RW];
#pragma unroll
        for (int rr = 0; rr < RW; rr++)
            if ((uint32_t)rr < c.rw) gv_w<F>(s, c.o0 + (uint32_t)rr * row_bytes + bl * S, part, tab, w[rr]);
#pragma unroll
        for (int m = 0; m < MT; m++) {
            if (m >= (int)nm) continue;
            GvA x;
            gv_a<F>(act, (uint32_t)m, c.c0 + bl, part, x);
#pragma unroll
            for (int rr = 0; rr < RW; rr++)
                if ((uint32_t)rr < c.rw) acc[rr][m] = gv_dot<F>(w[rr], x, acc[rr][m]);
        }
    }
}

// Codebook tables of the workgroup, strided over its threads.
template <int F>
NQ_HD void gv_fill_tables(uint64_t *t8, uint32_t *t4, uint32_t tid) {
    using TS = TabSpec<F>;
    if constexpr (TS::n8 > 0) {
        const uint64_t *g = TS::src8();
        for (uint32_t r = tid; r < (uint32_t)TS::n8; r += WG) t8[r] = g[r];
    }
    if constexpr (TS::n4 > 0) {
        const uint32_t *g = TS::src4();
        for (uint32_t r = tid; r < (uint32_t)TS::n4; r += WG) t4[r] = g[r];
    }
}

template <int F, int MT, bool ALDS, int RW>
__global__ __launch_bounds__(WG) void k_gemv(GvArgs a) {
    using TS = TabSpec<F>;
    __shared__ uint64_t t8[TS::n8 > 0 ? TS::n8 : 1];
    __shared__ uint32_t t4[TS::n4 > 0 ? TS::n4 : 1];
    extern __shared__ __attribute__((aligned(16))) uint32_t gv_lds[];
    if constexpr (TS::n8 + TS::n4 > 0) gv_fill_tables<F>(t8, t4, threadIdx.x);
    if constexpr (ALDS) gv_stage_act(a, gv_lds, threadIdx.x, WG);
    if constexpr (ALDS || TS::n8 + TS::n4 > 0) __syncthreads();
    const Tab tab{t8, t4, nullptr, nullptr, 0xFFFFFFFFu, 1u};
    const GvAct<ALDS> act{a.xq, gv_lds, a.K, a.kb, a.xrow, a.M};
    constexpr int NL = gv_nl<RW>();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t step = gridDim.x * GV_WAVES;
    uint32_t *lds = gv_lds + (ALDS ? gv_act_dw(a) : 0u) + wave * gv_wave_dw<RW>();
    const DevSrc src{a.wbase, a.wlast};
    uint32_t r = (blockIdx.x * GV_WAVES + wave) * a.rw, c0 = 0u;
    if (r >= a.rows) return;  // no workgroup barrier follows
    GvChunk cur = gv_chunk(a, r, c0);
    uint32_t v[NL][4];
    gv_issue<NL>(src, a.wlast, cur, lane, v);
    float acc[RW][MT], done[RW][MT];
#pragma unroll
    for (int rr = 0; rr < RW; rr++)
#pragma unroll
        for (int m = 0; m < MT; m++) acc[rr][m] = 0.0f;
    uint32_t done_r = 0xFFFFFFFFu, done_rw = 0u;  // finished rows whose sums are not stored yet
    for (;;) {
        wave_lds_sync();  // the previous chunk's readers are done
        gv_put<NL>(cur, a.wlast, lane, v, lds);
        wave_lds_sync();
        // Finished rows are stored here, before the next chunk's loads: the
        // memory counter is in order, so stores issued after them would
        // hold up the wait for them.
        if (done_r != 0xFFFFFFFFu) {
#pragma unroll
            for (int rr = 0; rr < RW; rr++)
#pragma unroll
                for (int m = 0; m < MT; m++)
                    if (lane == 63u && (uint32_t)rr < done_rw && m < (int)a.M)
                        a.y[(uint64_t)m * a.ldy + done_r + (uint32_t)rr] = done[rr][m];
            done_r = 0xFFFFFFFFu;
        }
        gv_advance(a, step, &r, &c0);
        const bool more = r < a.rows;
        GvChunk nxt = cur;
        if (more) {
            nxt = gv_chunk(a, r, c0);
            gv_issue<NL>(src, a.wlast, nxt, lane, v);  // in flight while this chunk is computed
        }
        gv_chunk_items<F, MT, RW>(LdsSrc{lds, 4u * (cur.g1 - cur.g0) + 3u}, cur, lane, a.M, a.row_bytes, act, tab,
                              acc);
        if (cur.c0 + cur.nb >= a.nbr) {
#pragma unroll
            for (int rr = 0; rr < RW; rr++)
#pragma unroll
                for (int m = 0; m < MT; m++) {
                    done[rr][m] = (uint32_t)rr < cur.rw ? wave_sum63(acc[rr][m]) : 0.0f;
                    acc[rr][m] = 0.0f;
                }
            done_r = cur.r;
            done_rw = cur.rw;
        }
        if (!more) break;
        cur = nxt;
    }
    if (done_r != 0xFFFFFFFFu) {
#pragma unroll
        for (int rr = 0; rr < RW; rr++)
#pragma unroll
            for (int m = 0; m < MT; m++)
                if (lane == 63u && (uint32_t)rr < done_rw && m < (int)a.M)
                    a.y[(uint64_t)m * a.ldy + done_r + (uint32_t)rr] = done[rr][m];
    }
}

// One activation row, single-round kernel: the lane's items i = lane,
// lane + 64, ... of the chunk (n items per row), each item's activation
// columns read once and used for every row of the chunk.  Each row's
// partial takes the items in the same order as gv_chunk_items.
template <int F, int RW, class Act, class Src>
NQ_HD void gv1_items1(const Src &ls, const GvChunk &c, uint32_t lane, uint32_t row_bytes, uint32_t n,
                      const Act &act, const Tab &tab, float (&acc)[RW][1]) {
    constexpr uint32_t IPB = GvItem<F>::IPB, S = (uint32_t)block_bytes(F);
    for (uint32_t i = lane; i < n; i += 64u) {
        const uint32_t bl = i / IPB, pt = i - bl * IPB;
        GvA x;
        gv_a<F>(act, 0u, c.c0 + bl, pt, x);
#pragma unroll
        for (int rr = 0; rr < RW; rr++)
            if ((uint32_t)rr < c.rw) {
                GvW w;
                gv_w<F>(ls, c.o0 + (uint32_t)rr * row_bytes + bl * S, pt, tab, w);
                acc[rr][0] = gv_dot<F>(w, x, acc[rr][0]);
            }
    }
}

// The activation row as the single-round kernel holds it in LDS: its kb
// q8_1 blocks as in memory (9 dwords each; block ab at dword 9 * ab), except
// that the workgroup (gv1_act_prep) replaces each block's binary16 sum
// half-word, which the product does not use, with the exact sum of its
// codes (|sum| <= 32 * 127, a signed 16-bit value).
struct GvActRaw {
    const uint32_t *lds;
    NQ_HD float block(uint32_t, uint32_t ab, uint32_t (&c)[8], int *S) const {
        const uint32_t *p = lds + 9u * ab;
#pragma unroll
        for (int j = 0; j < 8; j++) c[j] = p[1 + j];
        *S = (int)(int16_t)(uint16_t)(p[0] >> 16);
        return f16(p[0] & 0xFFFFu);
    }
};

// Formats whose product uses the activation blocks' code sums (gv_dot: a
// min, offset or delta term); the others skip gv1_act_prep.
template <int F>
constexpr bool gv_uses_sum() {
    return F == Q4_0 || F == Q4_1 || F == Q5_0 || F == Q5_1 || F == Q2_K || F == Q3_K || F == Q4_K ||
           F == Q5_K || F == Q6_K || F == TQ1_0 || F == TQ2_0 || F == Q1_0 || F == Q2_0 || F == IQ1_S;
}

// The exact code sums of the staged activation blocks t, t + nt, ... (thread
// t of nt), written over their sum half-words.
NQ_HD void gv1_act_prep(uint32_t *lds, uint32_t kb, uint32_t t, uint32_t nt) {
    for (uint32_t ab = t; ab < kb; ab += nt) {
        uint32_t *p = lds + 9u * ab;
        int s = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) s = dot4(ONES8, p[1 + j], s);
        p[0] = (p[0] & 0xFFFFu) | ((uint32_t)s << 16);
    }
}

// Waves per single-round workgroup at most (the hardware's 1024 threads).
constexpr uint32_t GV1_MAX_WAVES = 16u;

// s_waitcnt immediate for "at most n memory loads of this wave outstanding"
// (vmcnt in bits 3:0 and 15:14; the export and LDS counters left at their
// maxima, so they are not waited for).
constexpr uint32_t gv_vm_imm(uint32_t n) { return (n & 15u) | (7u << 4) | (15u << 8) | ((n >> 4) << 14); }
// s_waitcnt immediate for "no LDS access of this wave outstanding" (the
// memory and export counters at their maxima).
constexpr uint32_t GV_LGKM0_IMM = 15u | (7u << 4) | (0u << 8) | (3u << 14);

// Waits until at most x of the wave's memory loads are outstanding, with x
// rounded down to one of a few counts (waiting for fewer is always safe).
// x is wave-uniform.
__device__ inline void gv_wait_vm(uint32_t x) {
    if (x >= 32u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(32u));
    else if (x >= 16u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(16u));
    else if (x >= 12u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(12u));
    else if (x >= 8u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(8u));
    else if (x >= 6u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(6u));
    else if (x >= 4u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(4u));
    else if (x >= 3u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(3u));
    else if (x >= 2u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(2u));
    else if (x >= 1u)
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(1u));
    else
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(0u));
}

// LDS dwords the single-round kernel keeps for act_dw activation dwords
// (the wave regions after them start 16-byte aligned).
NQ_HD uint32_t gv1_act_region(uint32_t act_dw) { return (act_dw + 3u) & ~3u; }

// Phase 1 of a single-round workgroup: the activation blocks (act_dw dwords
// from a 16-byte aligned address: 16-byte loads to LDS, and the last
// act_dw mod 4 dwords by dword loads of wave 0) and the codebook tables
// (dword loads to LDS), spread over the workgroup's waves: load i of wave w
// moves group (or dword) 64 * (i * nw + w) + lane.
template <int F>
__device__ void gv1_stage(uint64_t *t8, uint32_t *t4, const uint32_t *xq, uint32_t *act, uint32_t act_dw,
                          uint32_t wave, uint32_t nw, uint32_t lane) {
    using TS = TabSpec<F>;
    const uint32_t ng = act_dw / 4u, rd = act_dw % 4u;
    for (uint32_t b = 64u * wave; b < ng; b += 64u * nw)
        if (b + lane < ng)
            __builtin_amdgcn_global_load_lds((const void *)(xq + 4u * (b + lane)),
                                             (__attribute__((address_space(3))) void *)(act + 4u * b), 16u, 0, 0);
    if (rd != 0u && wave == 0u && lane < rd)
        __builtin_amdgcn_global_load_lds((const void *)(xq + 4u * ng + lane),
                                         (__attribute__((address_space(3))) void *)(act + 4u * ng), 4u, 0, 0);
    if constexpr (TS::n8 > 0) {
        const uint32_t *g = (const uint32_t *)TS::src8();
        constexpr uint32_t nd = 2u * (uint32_t)TS::n8;
        for (uint32_t b = 64u * wave; b < nd; b += 64u * nw)
            if (b + lane < nd)
                __builtin_amdgcn_global_load_lds((const void *)(g + b + lane),
                                                 (__attribute__((address_space(3))) void *)((uint32_t *)t8 + b), 4u,
                                                 0, 0);
    }
    if constexpr (TS::n4 > 0) {
        const uint32_t *g = TS::src4();
        constexpr uint32_t nd = (uint32_t)TS::n4;
        for (uint32_t b = 64u * wave; b < nd; b += 64u * nw)
            if (b + lane < nd)
                __builtin_amdgcn_global_load_lds((const void *)(g + b + lane),
                                                 (__attribute__((address_space(3))) void *)(t4 + b), 4u, 0, 0);
    }
}

// Single-round variant: when every chunk of the launch can be resident at
// once, each wave takes exactly one chunk and the launch's waves cover all
// of them.  A chunk is RW whole rows (KS = 1) or, for long rows, one of KS
// parts of one row (RW = 1: part h holds blocks h * cb .. h * cb + cb - 1);
// the KS waves of a row sit in one workgroup and their row sums meet in
// LDS, added in part order.  A workgroup has nw = blockDim.x / 64 waves
// (up to 16), so that one LDS copy of the activation serves them all.
//
// Loads, all issued before any wait, in this order:
//  1. the workgroup's shared bytes, spread over its waves (gv1_stage): the
//     activation rows' q8_1 blocks as they are in memory (from LDS dword
//     0), and the codebook tables;
//  2. the wave's chunk, straight from global memory into the wave's LDS
//     region (16-byte loads to LDS, lane l of load k filling group 64k + l;
//     the launch's weight bytes start 16-byte aligned, as the host checks,
//     so every group is one aligned 16-byte load; a final group that passes
//     the last weight dword is loaded by its lane as the 16 bytes ending
//     there and shifted into place, gv_put's rule, so no load leaves the
//     payload's dwords).
// The memory counter completes in issue order, so waiting until no more
// loads are outstanding than the wave's chunk loads with an active lane
// (each of those is issued) means its phase-1 loads have landed; after a
// workgroup barrier every wave's have.  A wave then waits for its own chunk
// only: the compute of waves whose bytes arrived early overlaps the loads
// still in flight, and nothing is issued after the weight bytes.
template <int F, int MT, int RW, int KS>
__global__ __launch_bounds__(64 * GV1_MAX_WAVES) void k_gemv1(GvArgs a, uint32_t region_dw, uint32_t act_dw) {
    static_assert(KS == 1 || RW == 1, "a split row is a single-row chunk");
    using TS = TabSpec<F>;
    __shared__ uint64_t t8[TS::n8 > 0 ? TS::n8 : 1];
    __shared__ uint32_t t4[TS::n4 > 0 ? TS::n4 : 1];
    __shared__ float part[KS > 1 ? GV1_MAX_WAVES : 1][MT];
    extern __shared__ __attribute__((aligned(16))) uint32_t gv_lds[];
    const uint32_t nw = blockDim.x >> 6;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t cw = blockIdx.x * nw + wave;  // the wave's chunk
    const uint32_t r = KS == 1 ? cw * (uint32_t)RW : cw / (uint32_t)KS;
    const uint32_t h = KS == 1 ? 0u : cw % (uint32_t)KS;
    uint32_t *lds = gv_lds + gv1_act_region(act_dw) + wave * region_dw;
    const bool live = r < a.rows;
    gv1_stage<F>(t8, t4, a.xq, gv_lds, MT == 1 ? act_dw : 0u, wave, nw, lane);
    __builtin_amdgcn_sched_barrier(0);  // the shared bytes' loads stay ahead of the chunk's
    GvChunk c{};
    uint32_t issued = 0u;  // chunk loads with an active lane
    if (live) {
        c = gv_chunk(a, r, h * a.cb);
        const uint32_t ng = c.g1 - c.g0 + 1u;
        const bool tail = 4u * c.g1 + 3u > a.wlast;  // only the launch's last group can pass wlast
        const uint32_t nfull = tail ? ng - 1u : ng;
        issued = (nfull + 63u) / 64u;
        for (uint32_t k = 0; 64u * k < ng; k++) {
            const uint32_t j = 64u * k + lane;
            if (j < nfull)
                __builtin_amdgcn_global_load_lds((const void *)(a.wbase + 4u * (c.g0 + j)),
                                                 (__attribute__((address_space(3))) void *)(lds + 256u * k), 16u, 0,
                                                 NQ_NTL ? 2 : 0);
        }
        if (tail && lane == ((ng - 1u) & 63u)) {
            uint32_t v[1][4];
            const DevSrc src{a.wbase, a.wlast};
            src.load_stream4(a.wlast - 3u, v[0]);
            GvChunk one = c;
            one.g0 = c.g1;  // gv_put's view: the single group g1 at the region's group ng - 1
            gv_put<1>(one, a.wlast, 0u, v, lds + 4u * (ng - 1u));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    gv_wait_vm(issued);  // this wave's phase-1 loads have landed
    __builtin_amdgcn_s_barrier();  // and every wave's
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MT == 1 && gv_uses_sum<F>()) {
        // the activation blocks' code sums, once per workgroup, while the
        // chunks are still in flight
        gv1_act_prep(gv_lds, a.kb, threadIdx.x, blockDim.x);
        __builtin_amdgcn_s_waitcnt(GV_LGKM0_IMM);  // the LDS stores are done
        __builtin_amdgcn_s_barrier();              // every wave's
        __builtin_amdgcn_sched_barrier(0);
    }
    if (KS == 1 && !live) return;  // no workgroup barrier follows
    float acc[RW][MT];
#pragma unroll
    for (int rr = 0; rr < RW; rr++)
#pragma unroll
        for (int m = 0; m < MT; m++) acc[rr][m] = 0.0f;
    if (live) {
        __builtin_amdgcn_s_waitcnt(gv_vm_imm(0u));  // the chunk's loads to LDS have landed
        wave_lds_sync();                             // and the shifted last group's stores
        const Tab tab{t8, t4, nullptr, nullptr, 0xFFFFFFFFu, 1u};
        const Gv1Src<F> ls = gv_src<Gv1Src<F>>(lds, 4u * (c.g1 - c.g0) + 3u);
        if constexpr (MT == 1)
            gv1_items1<F, RW>(ls, c, lane, a.row_bytes, c.nb * GvItem<F>::IPB, GvActRaw{gv_lds}, tab, acc);
        else
            gv_chunk_items<F, MT, RW>(ls, c, lane, a.M, a.row_bytes, GvAct<false>{a.xq, nullptr, a.K, a.kb, a.xrow, a.M},
                                      tab, acc);
    }
    if constexpr (KS == 1) {
#pragma unroll
        for (int rr = 0; rr < RW; rr++)
#pragma unroll
            for (int m = 0; m < MT; m++) {
                const float v = wave_sum63(acc[rr][m]);
                if (lane == 63u && (uint32_t)rr < c.rw && m < (int)a.M)
                    a.y[(uint64_t)m * a.ldy + r + (uint32_t)rr] = v;
            }
    } else {
        // every wave of the workgroup reaches the barrier; part 0's wave adds
        // the other parts' sums in part order and stores the row
        float v[MT];
#pragma unroll
        for (int m = 0; m < MT; m++) v[m] = wave_sum63(acc[0][m]);
        if (h != 0u && lane == 63u) {
#pragma unroll
            for (int m = 0; m < MT; m++) part[wave][m] = v[m];
        }
        __syncthreads();
        if (h == 0u && live && lane == 63u) {
#pragma unroll
            for (int m = 0; m < MT; m++) {
                float t = v[m];
#pragma unroll
                for (int j = 1; j < KS; j++) t += part[wave + (uint32_t)j][m];
                if (m < (int)a.M) a.y[(uint64_t)m * a.ldy + r] = t;
            }
        }
    }
}

// Host description of one product call.
struct GvLaunch {
    const uint8_t *w;   // device weight payload [N, K]
    uint64_t N, K, M;
    const uint8_t *xq;  // device q8_1 activation blocks [M, K / 32]
    float *y;           // device output [M, N]
    uint32_t cus;       // compute units of the device
};

struct Q81Launch {
    const void *x;
    uint64_t nblocks;
    uint32_t *blocks;
    uint32_t *status;
};

// Whole rows a chunk holds: 4 or 2 when they fit one chunk, else 1.
inline uint32_t gv_rows_per_chunk(uint64_t row_bytes) {
    return 4 * row_bytes <= gv_chunk_bytes<4>() ? 4u : 2 * row_bytes <= gv_chunk_bytes<2>() ? 2u : 1u;
}

// Activation staged in LDS when its codes, scales and sums fit the budget.
inline bool gv_act_in_lds(uint64_t M, uint64_t K) { return M * (K + K / 32 * 8) <= GV_ACT_LDS_MAX; }

template <int F>
GvArgs gv_args(const GvLaunch &L, uint64_t r0, uint64_t rows) {
    constexpr uint64_t S = (uint64_t)block_bytes(F);
    const uint64_t nbr = L.K / (uint64_t)block_values(F), row_bytes = nbr * S;
    const uint8_t *start = L.w + r0 * row_bytes;
    GvArgs a;
    a.wbase = (const uint32_t *)((uintptr_t)start & ~(uintptr_t)3);
    a.wmis = (uint32_t)((uintptr_t)start & 3u);
    a.wlast = (uint32_t)((a.wmis + rows * row_bytes - 1) / 4);
    a.xq = (const uint32_t *)L.xq;
    a.y = L.y + r0;
    a.rows = (uint32_t)rows;
    a.row_bytes = (uint32_t)row_bytes;
    a.K = (uint32_t)L.K;
    a.kb = (uint32_t)(L.K / 32);
    a.xrow = (uint32_t)(L.K / 32 * 9);
    a.ldy = (uint32_t)L.N;
    a.M = (uint32_t)L.M;
    a.nbr = (uint32_t)nbr;
    // four or two whole rows per chunk when they fit; else chunks of at
    // most the single-row chunk bytes (every block is at most 292 bytes),
    // the row's chunks as even as whole blocks allow
    a.rw = gv_rows_per_chunk(row_bytes);
    const uint64_t cmax = (a.rw > 1u ? gv_chunk_bytes<2>() : gv_chunk_bytes<1>()) / S;
    const uint64_t nch = (nbr + cmax - 1) / cmax;
    a.cb = (uint32_t)((nbr + nch - 1) / nch);
    return a;
}

// LDS bytes of a launch: the staged activation (when in LDS) and the waves' regions.
inline uint32_t gv_lds_bytes(const GvArgs &a, bool alds) {
    return 4u * ((alds ? gv_act_dw(a) : 0u) + GV_WAVES * (a.rw > 1u ? gv_wave_dw<2>() : gv_wave_dw<1>()));
}

// Workgroups of a launch: as many as the device keeps resident (the waves
// persist), and no more than the row groups (rw rows each) need.
inline uint32_t gv_grid(const GvArgs &a, uint32_t resident) {
    const uint64_t groups = (a.rows + a.rw - 1) / a.rw, need = (groups + GV_WAVES - 1) / GV_WAVES;
    return (uint32_t)(need < resident ? need : resident);
}

// Rows per launch: every weight byte offset of a launch fits 32 bits.
template <int F>
uint64_t gv_max_rows(const GvLaunch &L) {
    return 0xFFFFFFF0ull / (L.K / (uint64_t)block_values(F) * (uint64_t)block_bytes(F));
}

template <int F, int MT, bool ALDS, int RW>
int launch_gemv_rw(const GvLaunch &L, hipStream_t stream) {
    const uint64_t max_rows = gv_max_rows<F>(L);
    for (uint64_t r0 = 0; r0 < L.N;) {
        const uint64_t rows = L.N - r0 < max_rows ? L.N - r0 : max_rows;
        const GvArgs a = gv_args<F>(L, r0, rows);
        const uint32_t lds = gv_lds_bytes(a, ALDS);
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k_gemv<F, MT, ALDS, RW>, WG, lds) !=
                hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        const uint32_t grid = gv_grid(a, (uint32_t)per_cu * L.cus);
        hipLaunchKernelGGL((k_gemv<F, MT, ALDS, RW>), dim3(grid), dim3(WG), lds, stream, a);
        if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
        r0 += rows;
    }
    return 0;
}

// The rows-per-chunk count is a template parameter: it fixes the registers
// the items hold.
template <int F, int MT, bool ALDS>
int launch_gemv_lds(const GvLaunch &L, hipStream_t stream) {
    const uint64_t row_bytes = L.K / (uint64_t)block_values(F) * (uint64_t)block_bytes(F);
    switch (gv_rows_per_chunk(row_bytes)) {
    case 4: return launch_gemv_rw<F, MT, ALDS, 4>(L, stream);
    case 2: return launch_gemv_rw<F, MT, ALDS, 2>(L, stream);
    default: return launch_gemv_rw<F, MT, ALDS, 1>(L, stream);
    }
}

template <int F, int MT>
int launch_gemv_mt(const GvLaunch &L, hipStream_t stream) {
    return gv_act_in_lds(L.M, L.K) ? launch_gemv_lds<F, MT, true>(L, stream) : launch_gemv_lds<F, MT, false>(L, stream);
}

#ifndef NQ_GV1
#define NQ_GV1 1
#endif

// LDS dwords of a single-round wave region for chunks of chunk_bytes bytes:
// the 16-byte groups such a chunk can span at any start offset, plus one
// group of padding.
inline uint32_t gv1_region_dw(uint64_t chunk_bytes) {
    return 4u * (uint32_t)((15u + chunk_bytes + 15u) / 16u + 1u);
}

// Rows per chunk of the single-round launch, candidate k (0..2) in order of
// preference: the fewest rows that fit (more, smaller chunks: less compute
// per wave once its bytes are in), except that more than one activation row
// takes two or three rows first (each activation read then serves every row
// of the chunk) when two-row chunks still give every SIMD two waves.
inline uint32_t gv1_candidate(uint64_t N, uint64_t M, uint32_t cus, int k) {
    static const uint32_t few[3] = {1u, 2u, 3u}, more[3] = {2u, 3u, 1u};
    return M > 1 && N / 2 >= 8u * (uint64_t)cus ? more[k] : few[k];
}

// Parts per row tried first for single-row chunks of one activation row: 2
// when a row holds more than 64 items (a lane would take several items of
// the row in turn) and at least two blocks, and either the rows are long
// (K >= 8192) or whole rows would give fewer than 16 waves per compute
// unit; else 1.  Measured on eight formats: the split gains 3-9% at
// [4096, 14336] for q4_k, q4_0, q2_k and iq2_xxs (loses up to 6% for
// mxfp4) and 5-10% at [1024, 4096], but loses 7-17% at [4096, 4096].
inline uint32_t gv1_parts(uint64_t N, uint64_t nbr, uint32_t ipb, uint64_t K, uint32_t cus) {
    return nbr >= 2u && nbr * ipb > 64u && (K >= 8192u || N < 16u * (uint64_t)cus) ? 2u : 1u;
}

// A single-round launch: rows per chunk (0: none), parts per row, blocks per
// chunk row, waves per workgroup, wave region and activation dwords, LDS
// bytes per workgroup and workgroups.
struct Gv1Plan {
    uint32_t rw, ks, cb, nw, region_dw, act_dw, lds, grid;
};

constexpr uint32_t GV1_LDS_MAX = 163840u;  // LDS bytes of a compute unit (and of one workgroup at most)

// The single-round plan of a launch of N rows of nbr blocks of S bytes (ipb
// items each) starting at address w, with M activation rows of K values at
// address xq, on `cus` compute units; per_cu(rw, ks, nw, lds) gives the
// workgroups of nw waves of that kernel a compute unit holds at once with
// that much dynamic LDS.  With one activation row (staged in LDS, one copy
// per workgroup), for each candidate (rows per chunk, and single-row chunks
// split in parts first) it takes the most workgroups per compute unit,
// g = 8 .. 1, whose waves per workgroup, ceil(chunks / (cus * g)) (even for
// split rows), stay within 16 and whose workgroups all fit at once: the
// smallest workgroups, whose barrier waits on the fewest waves (measured
// 0-13% faster than the largest that fit, at no loss); with several
// activation rows (read from global memory) workgroups have four waves and
// rows are not split.
// None (rw = 0) when the weight bytes or the activation do not start 16-byte
// aligned, the launch holds fewer than 16 bytes or more than 32-bit byte
// offsets reach (max_rows), or nothing fits.
template <class PerCu>
Gv1Plan gv1_plan(uint64_t N, uint64_t nbr, uint32_t S, uint32_t ipb, uint64_t M, uint64_t K, uint64_t max_rows,
                 uintptr_t w, uintptr_t xq, uint32_t cus, PerCu per_cu) {
    Gv1Plan p{0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    const uint64_t row_bytes = nbr * S, act_dw = M == 1u ? (K / 32u) * 9u : 0u;
    const uint64_t act_bytes = 4u * (uint64_t)gv1_act_region((uint32_t)act_dw);
    if (!NQ_GV1 || (w & 15u) != 0u || (xq & 15u) != 0u || N > max_rows || N * row_bytes < 16u || cus == 0u ||
        act_bytes > GV1_LDS_MAX)
        return p;
    for (int k = 0; k < 3; k++) {
        const uint32_t rw = gv1_candidate(N, M, cus, k);
        for (uint32_t ks = rw == 1u && M == 1u ? gv1_parts(N, nbr, ipb, K, cus) : 1u; ks >= 1u; ks /= 2u) {
            const uint64_t cb = (nbr + ks - 1u) / ks;
            const uint32_t region = gv1_region_dw(ks == 1u ? rw * row_bytes : cb * S);
            const uint64_t chunks = ks == 1u ? (N + rw - 1) / rw : N * ks;
            for (uint32_t gi = 8u; gi >= 1u; gi--) {
                uint64_t g = gi;
                uint64_t nw = (chunks + (uint64_t)cus * g - 1u) / ((uint64_t)cus * g);
                nw += nw % ks;
                if (M > 1u) {  // activation read from global memory: four-wave workgroups
                    if (gi < 8u) break;
                    nw = GV_WAVES;
                    g = (chunks + nw * cus - 1u) / (nw * cus);
                }
                if (nw > GV1_MAX_WAVES) continue;
                const uint64_t lds = act_bytes + 4u * nw * region;
                if (lds > GV1_LDS_MAX) continue;
                if ((uint64_t)per_cu(rw, ks, (uint32_t)nw, (uint32_t)lds) < g) continue;
                p.rw = rw;
                p.ks = ks;
                p.cb = (uint32_t)cb;
                p.nw = (uint32_t)nw;
                p.region_dw = region;
                p.act_dw = (uint32_t)act_dw;
                p.lds = (uint32_t)lds;
                p.grid = (uint32_t)((chunks + nw - 1u) / nw);
                return p;
            }
        }
    }
    return p;
}

template <int F, int MT, int RW, int KS>
int gv1_per_cu(uint32_t nw, uint32_t lds) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k_gemv1<F, MT, RW, KS>, 64 * (int)nw,
                                                     lds) != hipSuccess)
        return 0;
    return per_cu;
}

// The single-round launch when its plan exists; -1 (nothing launched) when not.
template <int F, int MT>
int launch_gemv1(const GvLaunch &L, hipStream_t stream) {
    const uint64_t nbr = L.K / (uint64_t)block_values(F);
    const Gv1Plan p = gv1_plan(L.N, nbr, (uint32_t)block_bytes(F), GvItem<F>::IPB, L.M, L.K, gv_max_rows<F>(L),
                               (uintptr_t)L.w, (uintptr_t)L.xq, L.cus,
                               [](uint32_t rw, uint32_t ks, uint32_t nw, uint32_t lds) {
                                   return ks == 2u   ? gv1_per_cu<F, MT, 1, 2>(nw, lds)
                                          : rw == 1u ? gv1_per_cu<F, MT, 1, 1>(nw, lds)
                                          : rw == 2u ? gv1_per_cu<F, MT, 2, 1>(nw, lds)
                                                     : gv1_per_cu<F, MT, 3, 1>(nw, lds);
                               });
    if (p.rw == 0u) return -1;
    GvArgs a = gv_args<F>(L, 0, L.N);
    a.rw = p.rw;
    a.cb = p.cb;
    const dim3 grid(p.grid), block(64u * p.nw);
    if (p.ks == 2u)
        hipLaunchKernelGGL((k_gemv1<F, MT, 1, 2>), grid, block, p.lds, stream, a, p.region_dw, p.act_dw);
    else if (p.rw == 1u)
        hipLaunchKernelGGL((k_gemv1<F, MT, 1, 1>), grid, block, p.lds, stream, a, p.region_dw, p.act_dw);
    else if (p.rw == 2u)
        hipLaunchKernelGGL((k_gemv1<F, MT, 2, 1>), grid, block, p.lds, stream, a, p.region_dw, p.act_dw);
    else
        hipLaunchKernelGGL((k_gemv1<F, MT, 3, 1>), grid, block, p.lds, stream, a, p.region_dw, p.act_dw);
    return hipGetLastError() != hipSuccess ? 9 : 0;  // NQ_ERR_HIP
}

template <int F, int MT>
int launch_gemv_m(const GvLaunch &L, hipStream_t s) {
    const int st = launch_gemv1<F, MT>(L, s);
    return st >= 0 ? st : launch_gemv_mt<F, MT>(L, s);
}

template <int F>
int launch_gemv_f(const GvLaunch &L, hipStream_t s) {
    if (L.M <= 1) return launch_gemv_m<F, 1>(L, s);
    if (L.M <= 2) return launch_gemv_m<F, 2>(L, s);
    if (L.M <= 4) return launch_gemv_m<F, 4>(L, s);
    return launch_gemv_m<F, 8>(L, s);
}

}  // namespace nq
