// nq_gemm.h -- batched products (many activation rows) of packed gguf_*
// weights with q8_1 activations on the 8-bit integer matrix cores.
//
// NInfer "tensor-formats" page, GGUF linear operations: the activation is
// quantized to ggml q8_1 blocks (one binary16 scale per 32 values) and the
// product accumulates in FP32.  The value each weight stands for is the one
// the format's decoder gives (DequantizePacked decoding specification,
// "Packed layouts and decoding" and "Mathematical decoding rules").
//
// Spans.  Every 32 consecutive values of a weight row (a span; no span
// crosses a block) are rewritten as 32 signed 8-bit codes c with, per half of
// 16 values (or per span for formats with one scale per 32 values), a scale
// ws and an offset ow such that w = ws * c + ow.  Then, with an activation
// block's scale d, codes q and exact half sums S_h,
//     sum over the span of w * d * q = d * sum_h (ws_h * I_h + ow_h * S_h),
// I_h = sum of c * q over the half (exact integers).  The I_h come from
// v_mfma_i32_16x16x32_i8 (a 16 x 16 tile of exact 32-term integer dot
// products); scales with 16-value halves take two MFMAs per span, each with
// the activation codes of the other half set to zero.  The scaling is done
// in binary32, per span and half:
//     acc = fma(RN(ws_h * d), I_h, acc)
// and, for the five affine formats (q4_1, q5_1, q2_k, q4_k, q5_k), the
// offset terms ow_h * (d * S_h) of a K step (d * S_h is exact: at most 11 by
// 12 significant bits) are added four spans at a time by
// v_mfma_f32_16x16x4_f32, the binary32 matrix instruction, into the same
// accumulators; for the other formats ws * c equals the decoded weight
// exactly.  Every gguf format
// has a rewrite.
//
// Tiling.  A workgroup (4 waves) owns a tile of 128 weight rows by 64
// activation rows and walks K in steps of 256 values (128 on grids of more
// than two 64-row tiles per compute unit, and with K split over five
// eighths to two such tiles per compute unit: half the LDS, so more
// workgroups share a compute unit and hide each other's staging): its
// threads rewrite the step's weight spans into LDS (codes, scales, offsets)
// and copy the activation codes, scales and d * S terms next to them; then
// each wave
// computes a 64 x 32 sub-tile, span by span, in a fixed order, so every run
// of a launch shape gives the same bits.  Tiles that share weight rows are
// given to workgroups of one XCD (workgroups go to the 8 XCDs in turn), so
// the weight bytes come from one L2.  With a workspace, shapes with few
// tiles and long K split K over workgroups (partial outputs summed in split
// order by a second launch), and large batches have the weight rewritten
// once per call so that the tiles copy it (gm_plan).  Without offset terms
// the step length leaves every output the same sum in the same order; the
// affine formats add their offset terms once per step, so the two step
// lengths round them in a different order.
#pragma once

#include "nq_gemv.h"

namespace nq {

constexpr uint32_t GM_BN = 128;            // weight rows per tile
constexpr uint32_t GM_BM = 64;             // activation rows per tile (32 for batches of at most 32 rows)
constexpr uint32_t GM_SP = 8;              // spans per K step (256 values; 4 on large grids, gm_plan)
constexpr uint64_t GM_MAX_MROWS = 1ull << 16;  // activation rows per launch

// Activation rows per launch for K columns: at most GM_MAX_MROWS, and few
// enough that byte offsets into the launch's q8_1 rows (K / 32 * 36 bytes
// each) fit 32 bits.
inline uint64_t gm_max_mrows(uint64_t K) {
    const uint64_t by_bytes = (1ull << 32) / (K / 32u * 36u);
    return by_bytes < GM_MAX_MROWS ? by_bytes : GM_MAX_MROWS;
}
constexpr uint64_t GM_MIN_M = 5;  // fewer activation rows take the single-row kernel (faster there)
#ifndef NQ_GM_REWRITE_M
#define NQ_GM_REWRITE_M 256
#endif
constexpr uint64_t GM_REWRITE_ONCE_M = NQ_GM_REWRITE_M;  // more activation rows: the weight is rewritten once per call

// one scale per 16 values
NQ_HD constexpr bool gm_u16(int f) {
    return f == Q2_K || f == Q3_K || f == Q6_K || f == IQ2_XS || f == IQ2_S || f == IQ1_M || f == NVFP4_GGUF;
}
// a code-independent term
NQ_HD constexpr bool gm_aff(int f) { return f == Q4_1 || f == Q5_1 || f == Q2_K || f == Q4_K || f == Q5_K; }

// Activation rows per tile: 16 for batches of at most 16 rows, 32 for at
// most 32, else 64.
NQ_HD uint32_t gm_bm(uint64_t M) { return M <= 16u ? 16u : M <= 32u ? 32u : GM_BM; }

// Wave layout of a tile: each of the 4 waves computes NI 16-row weight
// subtiles by MJ 16-row activation subtiles; WN waves side by side along the
// 128 weight rows, WM along the activation rows.  (NI, MJ) = (4, 2): 64
// activation rows, (4, 1): 32, (2, 1): 16.
template <int NI, int MJ>
struct GmShape {
    static constexpr uint32_t WN = 8u / (uint32_t)NI, WM = 4u / WN, BM = 16u * (uint32_t)MJ * WM;
    static_assert(WN * WM == 4u && 16u * (uint32_t)NI * WN == 128u, "4 waves over 128 weight rows");
    NQ_HD static uint32_t nb(uint32_t w) { return 16u * (uint32_t)NI * (w % WN); }
    NQ_HD static uint32_t mb(uint32_t w) { return 16u * (uint32_t)MJ * (w / WN); }
};

template <int F, int BMT = 64, int SPT = 8>
struct GmFmt {
    static constexpr uint32_t BM = (uint32_t)BMT;  // activation rows per tile
    static constexpr uint32_t SP = (uint32_t)SPT;  // spans per K step
    static constexpr uint32_t CSW = 8u * SP + 4u;  // LDS dwords per code row (the step's codes + 16 bytes)
    static constexpr bool U16 = gm_u16(F);
    static constexpr bool AFF = gm_aff(F);
    // formats with a span rewrite (every gguf format)
    static constexpr bool OK = F != NVFP4_DIV;
    static constexpr uint32_t NH = U16 ? 2u : 1u;  // scales per span
    static constexpr uint32_t SPB = (uint32_t)block_values(F) / 32u;  // spans per block
    // LDS layout (dwords): weight codes [128][CSW], scales [SP][NH][128],
    // offsets [SP][NH][128] (affine formats), activation codes [BM][CSW],
    // scales [SP][BM], d * S terms [SP][NH][BM] (affine formats)
    static constexpr uint32_t WS = GM_BN * CSW;
    static constexpr uint32_t WO = WS + SP * NH * GM_BN;
    static constexpr uint32_t XC = WO + (AFF ? SP * NH * GM_BN : 0u);
    static constexpr uint32_t XD = XC + BM * CSW;
    static constexpr uint32_t XT = XD + SP * BM;
    static constexpr uint32_t DW = XT + (AFF ? SP * NH * BM : 0u);
};

struct GmArgs {
    const uint32_t *wbase;  // weight bytes of this launch's first row, aligned down to 4 bytes
    uint32_t wmis;          // that row's start - wbase (0..3)
    uint32_t wlast;         // last dword holding weight bytes of this launch, from wbase
    const uint32_t *xq;     // q8_1 blocks of this launch's first activation row (9 dwords each)
    float *y;               // output of this launch's first activation and weight row
    uint32_t rows;          // weight rows in this launch
    uint32_t row_bytes;     // bytes per weight row
    uint32_t kspans;        // K / 32
    uint32_t xrow;          // dwords per activation row, K / 32 * 9
    uint32_t ldy;           // N
    uint32_t M;             // activation rows in this launch
    uint32_t mt;            // activation-row tiles
    uint32_t bm;            // activation rows per tile
    uint32_t xq8, xr8;      // workgroups / 8 and workgroups mod 8
    uint32_t nsplit;        // K splits (1: none)
    uint32_t sps;           // K steps per split
    uint64_t ysplit;        // elements between two splits' partial outputs (M * N)
    // the weight rewritten once per call (null: rewritten per tile): codes of
    // this launch's first row (K bytes per row), and its scales and offsets
    // (value (span t, half h, row n) at (t * NH + h) * N + n from these)
    const uint32_t *cw;
    const float *cs, *co;
};

// A span rewritten: 32 codes (8 dwords, value order) and per half its scale
// and offset.
struct GmSpan {
    uint32_t c[8];
    float ws[2];
    float ow[2];
};

// Weight source in global memory: dword loads of any window length from a
// 4-byte-aligned base (16-byte vector loads, then 8 and 4 bytes); `last` is
// the last dword holding payload bytes, and a window's extra dword is clamped
// to it.
struct GmSrc {
    const uint32_t *base;
    uint32_t last;
    template <int N>
    NQ_HD void load(uint32_t i, uint32_t (&r)[N]) const {
        const uint32_t *p = base + i;
#pragma unroll
        for (int k = 0; k + 4 <= N; k += 4) {
            const u32x4a4 v = *(const u32x4a4 *)(p + k);
            r[k] = v.x;
            r[k + 1] = v.y;
            r[k + 2] = v.z;
            r[k + 3] = v.w;
        }
        constexpr int k2 = N / 4 * 4;
        if constexpr (N - k2 >= 2) {
            const u32x2a4 v = *(const u32x2a4 *)(p + k2);
            r[k2] = v.x;
            r[k2 + 1] = v.y;
        }
        if constexpr ((N - k2) % 2 == 1) r[N - 1] = p[N - 1];
    }
    NQ_HD uint32_t dw(uint32_t i) const { return base[i]; }
    NQ_HD uint32_t dwx(uint32_t i) const { return base[i < last ? i : last]; }
};

// Span p of the block at byte offset bo.
template <int F, class Src>
NQ_HD void gm_span(const Src &s, uint32_t bo, uint32_t p, const Tab &tab, GmSpan &o) {
    constexpr uint32_t LO4 = 0x0F0F0F0Fu;
    o.ow[0] = o.ow[1] = 0.0f;
    if constexpr (F == Q4_K || F == Q5_K) {
        // sub-block p: nibble plane p mod 2 of the 32 code bytes of pair p / 2
        // (q4_k at 16, q5_k at 48), q5_k's fifth bit from bit p of bytes 16..47;
        // w = RN32(d * sc) * v - RN32(dmin * m)
        uint32_t h[4], q[8];
        window<4>(s, bo, h);
        window<8>(s, bo + (F == Q4_K ? 16u : 48u) + 32u * (p >> 1), q);
        const float d = f16(h[0] & 0xFFFFu), dmin = f16(h[0] >> 16);
        const uint32_t hs[3] = {h[1], h[2], h[3]};
        uint32_t sc, mn;
        kq_scale_min(hs, p, &sc, &mn);
        o.ws[0] = o.ws[1] = M(d, (float)sc);
        o.ow[0] = o.ow[1] = -M(dmin, (float)mn);
        const uint32_t sh = 4u * (p & 1u);
        if constexpr (F == Q4_K) {
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = (q[j] >> sh) & LO4;
        } else {
            uint32_t qh[8];
            window<8>(s, bo + 16u, qh);
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = ((q[j] >> sh) & LO4) | (((qh[j] >> p) & 0x01010101u) << 4);
        }
    } else if constexpr (F == Q6_K) {
        // values 32p + i: with h = p / 4, c = p mod 4, the low 4 bits are
        // nibble c / 2 of byte 64h + 32(c mod 2) + i, the high 2 bits bits 2c
        // of byte 128 + 32h + i; the 16-value sub-blocks 2p and 2p + 1 take the
        // signed scale bytes 192 + 2p and 193 + 2p; w = RN32(d * sc) * (v - 32)
        const uint32_t hh = p >> 2, c = p & 3u;
        uint32_t ql[8], qh[8];
        window<8>(s, bo + 64u * hh + 32u * (c & 1u), ql);
        window<8>(s, bo + 128u + 32u * hh, qh);
        const uint32_t sw = u16_at(s, bo + 192u + 2u * p);
        const float d = f16(u16_at(s, bo + 208u));
        o.ws[0] = M(d, (float)(int8_t)(sw & 0xFFu));
        o.ws[1] = M(d, (float)(int8_t)(sw >> 8));
#pragma unroll
        for (int j = 0; j < 8; j++)
            o.c[j] = bsub(((ql[j] >> (4u * (c >> 1))) & LO4) | (((qh[j] >> (2u * c)) & 0x03030303u) << 4), 0x20202020u);
    } else {
        // the single-row kernel's item p (whole span), then its codes made
        // signed and its scales and offsets sorted into halves
        GvW w;
        gv_w<F>(s, bo, p, tab, w);
        if constexpr (F == Q8_0 || F == Q8_1 || F == Q8_K || F == IQ4_NL || F == MXFP4 || F == IQ4_XS) {
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = w.q[j];
            o.ws[0] = o.ws[1] = w.f[0];
        } else if constexpr (F == TQ1_0) {
            // codes digit - 1
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = bsub(w.q[j], 0x01010101u);
            o.ws[0] = o.ws[1] = w.f[0];
        } else if constexpr (F == Q4_0) {
            // codes v - 8 (the item's words: the low nibbles, then the high)
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = bsub(w.q[j], 0x08080808u);
            o.ws[0] = o.ws[1] = w.f[0];
        } else if constexpr (F == Q4_1 || F == Q5_1) {
            // w = d * v + m
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = w.q[j];
            o.ws[0] = o.ws[1] = w.f[0];
            o.ow[0] = o.ow[1] = w.f[1];
        } else if constexpr (F == Q5_0 || F == TQ2_0 || F == Q2_0 || F == Q3_K) {
            // w = scale * (v - o), o = 16, 1, 1, 4
            constexpr uint32_t O = F == Q5_0 ? 0x10101010u : F == Q3_K ? 0x04040404u : 0x01010101u;
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = bsub(w.q[j], O);
            o.ws[0] = w.f[0];
            o.ws[1] = F == Q3_K ? w.f[1] : w.f[0];
        } else if constexpr (F == Q1_0) {
            // code 2b - 1: byte 0xFF - 0xFE b
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = ~(w.q[j] * 0xFEu);
            o.ws[0] = o.ws[1] = w.f[0];
        } else if constexpr (F == Q2_K) {
            // two sub-blocks: w = RN32(d * s) * v - RN32(dmin * m)
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = w.q[j];
            o.ws[0] = w.f[0];
            o.ow[0] = -w.f[1];
            o.ws[1] = w.f[2];
            o.ow[1] = -w.f[3];
        } else if constexpr (F == NVFP4_GGUF) {
            // two 16-value groups, doubled E2M1 codes, half scales
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = w.q[j];
            o.ws[0] = w.f[0];
            o.ws[1] = w.f[1];
        } else if constexpr (F == IQ2_XXS || F == IQ3_XXS || F == IQ3_S || F == IQ2_XS || F == IQ2_S) {
            // grid bytes g (< 128) and the bytes n = g under the negative
            // signs: the signed value is g where n = 0 and -g where n = g
#pragma unroll
            for (int j = 0; j < 8; j++) o.c[j] = (w.q[j] ^ w.q[8 + j]) | bsub(0u, w.q[8 + j]);
            o.ws[0] = w.f[0];
            o.ws[1] = F == IQ2_XS || F == IQ2_S ? w.f[1] : w.f[0];
        } else if constexpr (F == IQ1_S || F == IQ1_M) {
            // grid bytes hold v + 1 (v in -1, 0, 1); w = scale * (v + delta),
            // delta = +-1/8: codes 8v + 8 delta = 8 g - 8 + 8 delta, scale / 8
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float dl = F == IQ1_S ? w.f[1] : w.f[2 + (j >> 1)];
                o.c[j] = bsub(w.q[j] << 3, dl < 0.0f ? 0x09090909u : 0x07070707u);
            }
            o.ws[0] = M(w.f[0], 0.125f);
            o.ws[1] = F == IQ1_M ? M(w.f[1], 0.125f) : o.ws[0];
        } else {
            static_assert(F < 0, "format without a span rewrite");
        }
    }
}

// Workgroup id -> (weight tile, activation tile, K split): ids go to the
// XCDs in turn (id mod 8); each XCD's ids take a contiguous range of
// numbers, and numbers run over K splits first, then activation tiles, so the
// work on one group of weight rows falls on one XCD.  A bijection of
// [0, grid).
NQ_HD void gm_tile(const GmArgs &a, uint32_t id, uint32_t *n0, uint32_t *m0, uint32_t *ks) {
    const uint32_t x = id & 7u, j = id >> 3;
    const uint32_t L = (x < a.xr8 ? x * (a.xq8 + 1u) : a.xr8 * (a.xq8 + 1u) + (x - a.xr8) * a.xq8) + j;
    const uint32_t T = L / a.nsplit;
    *ks = L - T * a.nsplit;
    *m0 = (T % a.mt) * a.bm;
    *n0 = (T / a.mt) * GM_BN;
}

// K step: the spans t0 .. t0+SP-1 of weight rows n0 .. n0+127, rewritten
// into LDS; thread tid takes items tid + WG r (r < SP / 2), item i = (row
// i / SP, span i mod SP).  The loads take no branch (an item past the
// launch's rows or past K reads the launch's first span and is then zeroed),
// so the items' loads are all in flight at once.
template <int F, int SP, class Src>
NQ_HD void gm_stage_w(const GmArgs &a, const Src &src, const Tab &tab, uint32_t n0, uint32_t t0, uint32_t tid,
                      uint32_t *lds) {
    using G = GmFmt<F, 64, SP>;
    constexpr uint32_t S = (uint32_t)block_bytes(F);
    constexpr uint32_t R = GM_BN * G::SP / (uint32_t)WG;
    static_assert(GM_BN * G::SP % (uint32_t)WG == 0, "whole items per thread");
    GmSpan o[R];
    bool ok[R];
#pragma unroll
    for (uint32_t r = 0; r < R; r++) {
        const uint32_t i = tid + (uint32_t)WG * r, n = i / G::SP, t = t0 + i % G::SP;
        ok[r] = n0 + n < a.rows && t < a.kspans;
        const uint32_t nn = ok[r] ? n0 + n : 0u, tt = ok[r] ? t : 0u, b = tt / G::SPB;
        gm_span<F>(src, a.wmis + nn * a.row_bytes + b * S, tt - b * G::SPB, tab, o[r]);
    }
    float *ws = (float *)(lds + G::WS), *ow = (float *)(lds + G::WO);
#pragma unroll
    for (uint32_t r = 0; r < R; r++) {
        const uint32_t i = tid + (uint32_t)WG * r, n = i / G::SP, sp = i % G::SP;
        uint32_t *cw = lds + n * G::CSW + 8u * sp;
#pragma unroll
        for (int j = 0; j < 8; j++) cw[j] = ok[r] ? o[r].c[j] : 0u;
#pragma unroll
        for (uint32_t h = 0; h < G::NH; h++) {
            ws[(sp * G::NH + h) * GM_BN + n] = ok[r] ? o[r].ws[h] : 0.0f;
            if constexpr (G::AFF) ow[(sp * G::NH + h) * GM_BN + n] = ok[r] ? o[r].ow[h] : 0.0f;
        }
    }
}

// K step from the weight rewritten once per call: the same LDS contents as
// gm_stage_w, copied (two 16-byte loads of codes and the scales / offsets
// per item, no per-format work).
template <int F, int SP>
NQ_HD void gm_stage_wc(const GmArgs &a, uint32_t n0, uint32_t t0, uint32_t tid, uint32_t *lds) {
    using G = GmFmt<F, 64, SP>;
    constexpr uint32_t R = GM_BN * G::SP / (uint32_t)WG;
    uint32_t c[R][8];
    float sw[R][2], so[R][2];
    bool ok[R];
#pragma unroll
    for (uint32_t r = 0; r < R; r++) {
        const uint32_t i = tid + (uint32_t)WG * r, n = i / G::SP, t = t0 + i % G::SP;
        ok[r] = n0 + n < a.rows && t < a.kspans;
        const uint32_t nn = ok[r] ? n0 + n : 0u, tt = ok[r] ? t : 0u;
        // 32-bit byte offsets: a launch's codes and scales each span fewer
        // than 2^32 bytes (gm_max_rows, launch_gemm_mfma)
        const uint32_t *p = (const uint32_t *)((const uint8_t *)a.cw + (nn * a.kspans + tt) * 32u);
        const u32x4 v0 = *(const u32x4 *)p, v1 = *(const u32x4 *)(p + 4);
        c[r][0] = v0.x; c[r][1] = v0.y; c[r][2] = v0.z; c[r][3] = v0.w;
        c[r][4] = v1.x; c[r][5] = v1.y; c[r][6] = v1.z; c[r][7] = v1.w;
#pragma unroll
        for (uint32_t h = 0; h < G::NH; h++) {
            const uint32_t kb = ((tt * G::NH + h) * a.ldy + nn) * 4u;
            sw[r][h] = *(const float *)((const uint8_t *)a.cs + kb);
            so[r][h] = G::AFF ? *(const float *)((const uint8_t *)a.co + kb) : 0.0f;
        }
    }
    float *ws = (float *)(lds + G::WS), *ow = (float *)(lds + G::WO);
#pragma unroll
    for (uint32_t r = 0; r < R; r++) {
        const uint32_t i = tid + (uint32_t)WG * r, n = i / G::SP, sp = i % G::SP;
        uint32_t *cw = lds + n * G::CSW + 8u * sp;
#pragma unroll
        for (int j = 0; j < 8; j++) cw[j] = ok[r] ? c[r][j] : 0u;
#pragma unroll
        for (uint32_t h = 0; h < G::NH; h++) {
            ws[(sp * G::NH + h) * GM_BN + n] = ok[r] ? sw[r][h] : 0.0f;
            if constexpr (G::AFF) ow[(sp * G::NH + h) * GM_BN + n] = ok[r] ? so[r][h] : 0.0f;
        }
    }
}

// The per-call rewrite, item g of a launch: groups of 8 items are 8
// consecutive spans of one row (their codes 256 contiguous bytes), groups
// run over the rows first (row (g / 8) mod rows, spans 8 ((g / 8) / rows)
// + g mod 8); codes to cw (K bytes per row), scales and offsets to cs / co.
NQ_HD uint64_t gm_rewrite_items(uint32_t rows, uint32_t kspans) { return (uint64_t)rows * ((kspans + 7u) / 8u) * 8u; }

// Item g's span: its row n and span t (false past K), its codes stored to
// cw, its scales and offsets in o.
template <int F, class Src>
NQ_HD bool gm_rewrite_span(const GmArgs &a, const Src &src, const Tab &tab, uint64_t g, uint32_t *cw, uint32_t *n_out,
                           uint32_t *t_out, GmSpan &o) {
    using G = GmFmt<F>;
    const uint64_t g8 = g >> 3;
    const uint32_t n = (uint32_t)(g8 % a.rows), t = (uint32_t)(g8 / a.rows) * 8u + (uint32_t)(g & 7u);
    if (t >= a.kspans) return false;
    const uint32_t b = t / G::SPB;
    gm_span<F>(src, a.wmis + n * a.row_bytes + b * (uint32_t)block_bytes(F), t - b * G::SPB, tab, o);
    u32x4 *d = (u32x4 *)(cw + (uint64_t)n * a.kspans * 8u + (uint64_t)t * 8u);
    d[0] = u32x4{o.c[0], o.c[1], o.c[2], o.c[3]};
    d[1] = u32x4{o.c[4], o.c[5], o.c[6], o.c[7]};
    *n_out = n;
    *t_out = t;
    return true;
}

template <int F, class Src>
NQ_HD void gm_rewrite_item(const GmArgs &a, const Src &src, const Tab &tab, uint64_t g, uint32_t *cw, float *cs,
                           float *co) {
    using G = GmFmt<F>;
    GmSpan o;
    uint32_t n, t;
    if (!gm_rewrite_span<F>(a, src, tab, g, cw, &n, &t, o)) return;
#pragma unroll
    for (uint32_t h = 0; h < G::NH; h++) {
        cs[((uint64_t)t * G::NH + h) * a.ldy + n] = o.ws[h];
        if constexpr (G::AFF) co[((uint64_t)t * G::NH + h) * a.ldy + n] = o.ow[h];
    }
}

// K step, activation side: blocks t0 .. t0+SP-1 of activation rows m0 ..
// m0+BM-1 (codes, binary32 scale, and for the affine formats d times the
// exact code sum of each half); thread tid takes items tid + WG r, item i =
// (row i / SP, block i mod SP), loaded without branches as above.
template <int F, int BMT, int SP>
NQ_HD void gm_stage_x(const GmArgs &a, uint32_t m0, uint32_t t0, uint32_t tid, uint32_t *lds) {
    using G = GmFmt<F, BMT, SP>;
    // BM * SP items: whole multiples of the workgroup, or (16 rows) half of it
    constexpr uint32_t R = (G::BM * G::SP + (uint32_t)WG - 1u) / (uint32_t)WG;
    uint32_t c[R][8];
    float d[R];
    bool ok[R];
#pragma unroll
    for (uint32_t r = 0; r < R; r++) {
        const uint32_t i = tid + (uint32_t)WG * r, m = i / G::SP, t = t0 + i % G::SP;
        ok[r] = i < G::BM * G::SP && m0 + m < a.M && t < a.kspans;
        // a 32-bit byte offset: a launch's activation rows span fewer than
        // 2^32 bytes (gm_max_mrows)
        const uint32_t *p = (const uint32_t *)((const uint8_t *)a.xq +
                                               (ok[r] ? ((m0 + m) * a.xrow + t * 9u) * 4u : 0u));
        const u32x4a4 v0 = *(const u32x4a4 *)(p + 1), v1 = *(const u32x4a4 *)(p + 5);
        c[r][0] = v0.x; c[r][1] = v0.y; c[r][2] = v0.z; c[r][3] = v0.w;
        c[r][4] = v1.x; c[r][5] = v1.y; c[r][6] = v1.z; c[r][7] = v1.w;
        d[r] = f16(p[0] & 0xFFFFu);
    }
#pragma unroll
    for (uint32_t r = 0; r < R; r++) {
        const uint32_t i = tid + (uint32_t)WG * r, m = i / G::SP, sp = i % G::SP;
        if (i >= G::BM * G::SP) continue;  // (16-row tiles) threads past the tile's items
        const float dr = ok[r] ? d[r] : 0.0f;
        uint32_t *cx = lds + G::XC + m * G::CSW + 8u * sp;
#pragma unroll
        for (int j = 0; j < 8; j++) cx[j] = ok[r] ? c[r][j] : 0u;
        ((float *)(lds + G::XD))[sp * G::BM + m] = dr;
        if constexpr (G::AFF) {
            int S0 = 0, S1 = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                S0 = dot4(ONES8, c[r][j], S0);
                S1 = dot4(ONES8, c[r][4 + j], S1);
            }
            float *xt = (float *)(lds + G::XT);
            if constexpr (G::U16) {
                xt[(2u * sp) * G::BM + m] = dr * (float)S0;
                xt[(2u * sp + 1u) * G::BM + m] = dr * (float)S1;
            } else {
                xt[sp * G::BM + m] = dr * (float)(S0 + S1);
            }
        }
    }
}

// MFMA operands of span sp for a lane of wave w (sub-tile: weight rows
// GmShape::nb(w) + 16 i + .., activation rows GmShape::mb(w) + 16 j + ..): the
// lane supplies row lane mod 16 of each 16-row group, code bytes
// 8 (lane / 16) .. + 7 of the span.
template <int NI, int MJ>
struct GmOps {
    uint64_t A[NI];  // weight rows
    uint64_t B[MJ];  // activation rows
};

NQ_HD uint64_t lds_u64(const uint32_t *p) { return (uint64_t)p[0] | ((uint64_t)p[1] << 32); }

template <int F, int NI, int MJ, int SP>
NQ_HD void gm_ops(const uint32_t *lds, uint32_t w, uint32_t lane, uint32_t sp, GmOps<NI, MJ> &o) {
    using Sh = GmShape<NI, MJ>;
    using G = GmFmt<F, Sh::BM, SP>;
    const uint32_t r = lane & 15u, k = 8u * sp + 2u * (lane >> 4);
    const uint32_t nb = Sh::nb(w), mb = Sh::mb(w);
#pragma unroll
    for (int i = 0; i < NI; i++) o.A[i] = lds_u64(lds + (nb + 16u * (uint32_t)i + r) * G::CSW + k);
#pragma unroll
    for (int j = 0; j < MJ; j++) o.B[j] = lds_u64(lds + G::XC + (mb + 16u * (uint32_t)j + r) * G::CSW + k);
}

// Activation operand for half h of a span with 16-value scales: lanes 0-31
// hold code bytes 0-15, lanes 32-63 bytes 16-31; the other half is zeroed.
template <int F>
NQ_HD uint64_t gm_half(uint64_t b, uint32_t lane, uint32_t h) {
    if constexpr (GmFmt<F>::U16)
        return (lane >> 5) == h ? b : 0ull;
    else
        return b;
}

// Integer results of a span for one lane: I[h][i][j][e] is the dot product of
// weight row nb(w) + 16 i + 4 (lane / 16) + e with activation row
// mb(w) + 16 j + lane mod 16 over half h (or the whole span).
template <int F, int NI, int MJ>
struct GmI {
    int v[GmFmt<F>::NH][NI][MJ][4];
};

// The span's scaling into the lane's accumulators (fixed order: per output,
// the halves).  The affine formats' offset terms are added per K step by
// gm_offsets on the matrix cores.
template <int F, int NI, int MJ, int SP>
NQ_HD void gm_epi(const uint32_t *lds, uint32_t w, uint32_t lane, uint32_t sp, const GmI<F, NI, MJ> &I,
                  float (&acc)[NI][MJ][4]) {
    using Sh = GmShape<NI, MJ>;
    using G = GmFmt<F, Sh::BM, SP>;
    const uint32_t nb = Sh::nb(w) + 4u * (lane >> 4), mb = Sh::mb(w) + (lane & 15u);
    const float *ws = (const float *)(lds + G::WS);
    const float *xd = (const float *)(lds + G::XD);
    float d[MJ];
#pragma unroll
    for (int j = 0; j < MJ; j++) d[j] = xd[sp * G::BM + mb + 16u * (uint32_t)j];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        float sw[2][4];
#pragma unroll
        for (uint32_t h = 0; h < G::NH; h++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                sw[h][e] = ws[(sp * G::NH + h) * GM_BN + nb + 16u * (uint32_t)i + (uint32_t)e];
#pragma unroll
        for (int j = 0; j < MJ; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                float a = acc[i][j][e];
#pragma unroll
                for (uint32_t h = 0; h < G::NH; h++) a = __builtin_fmaf(sw[h][e] * d[j], (float)I.v[h][i][j][e], a);
                acc[i][j][e] = a;
            }
    }
}

// Offset terms of the affine formats for one K step: with k = span * NH +
// half, they add sum_k ow[k][n] * (d S)[k][m] to every output, a product of
// the [n, k] offsets and the [k, m] terms.  v_mfma_f32_16x16x4_f32 adds four
// k at a time into the accumulators (A[i][k]: lane l supplies row l mod 16,
// k = l / 16; B[k][j] likewise; the result has the int8 tiles' lane layout).
// Operands of quad q for a lane (k past the step's nk are zeros).
template <int F, int NI, int MJ, int SP>
NQ_HD void gm_offsets_ops(const uint32_t *lds, uint32_t w, uint32_t lane, uint32_t q, uint32_t nk, float (&A)[NI],
                          float (&B)[MJ]) {
    using Sh = GmShape<NI, MJ>;
    using G = GmFmt<F, Sh::BM, SP>;
    const uint32_t k = 4u * q + (lane >> 4), r = lane & 15u;
    const uint32_t nb = Sh::nb(w), mb = Sh::mb(w);
    const float *ow = (const float *)(lds + G::WO), *xt = (const float *)(lds + G::XT);
    const bool in = k < nk;
    const uint32_t kk = in ? k : 0u;
#pragma unroll
    for (int i = 0; i < NI; i++) A[i] = in ? ow[kk * GM_BN + nb + 16u * (uint32_t)i + r] : 0.0f;
#pragma unroll
    for (int j = 0; j < MJ; j++) B[j] = in ? xt[kk * G::BM + mb + 16u * (uint32_t)j + r] : 0.0f;
}

// The lane's outputs: y[m][n] for its NI x MJ x 4 (row, activation row)
// pairs inside the launch (with K splits: split ks's partial output).
template <int NI, int MJ>
NQ_HD void gm_store(const GmArgs &a, uint32_t n0, uint32_t m0, uint32_t ks, uint32_t w, uint32_t lane,
                    const float (&acc)[NI][MJ][4]) {
    using Sh = GmShape<NI, MJ>;
    const uint32_t nb = n0 + Sh::nb(w) + 4u * (lane >> 4), mb = m0 + Sh::mb(w) + (lane & 15u);
#pragma unroll
    for (int j = 0; j < MJ; j++) {
        const uint32_t m = mb + 16u * (uint32_t)j;
        if (m >= a.M) continue;
        float *yr = a.y + (uint64_t)ks * a.ysplit + (uint64_t)m * a.ldy;
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t n = nb + 16u * (uint32_t)i + (uint32_t)e;
                if (n < a.rows) yr[n] = acc[i][j][e];
            }
    }
}

typedef int gm_i32x4 __attribute__((ext_vector_type(4)));

// With 128-value K steps the LDS of four workgroups fits a compute unit;
// asking for four waves per SIMD keeps the kernels with a few more than 128
// VGPRs (q2_k, iq2_s, nvfp4) at that occupancy, at the cost of a few
// spilled registers (measured +3 to +16% for those three at 512 and 2048
// activation rows, the others unchanged).

template <int F, int NI, int MJ, int SP>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(SP == 4 ? 4 : 1))) void k_gemm(GmArgs a) {
    using Sh = GmShape<NI, MJ>;
    using G = GmFmt<F, Sh::BM, SP>;
    using TS = TabSpec<F>;
    __shared__ uint64_t t8[TS::n8 > 0 ? TS::n8 : 1];
    __shared__ uint32_t t4[TS::n4 > 0 ? TS::n4 : 1];
    __shared__ __attribute__((aligned(16))) uint32_t lds[G::DW];
    if constexpr (TS::n8 + TS::n4 > 0) gv_fill_tables<F>(t8, t4, threadIdx.x);
    const Tab tab{t8, t4, nullptr, nullptr, 0xFFFFFFFFu, 1u};
    const GmSrc src{a.wbase, a.wlast};
    uint32_t n0, m0, ks;
    gm_tile(a, blockIdx.x, &n0, &m0, &ks);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    float acc[NI][MJ][4];
#pragma unroll
    for (int i = 0; i < NI; i++)
#pragma unroll
        for (int j = 0; j < MJ; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) acc[i][j][e] = 0.0f;
    const uint32_t tb = ks * a.sps * G::SP, te0 = tb + a.sps * G::SP, te = te0 < a.kspans ? te0 : a.kspans;
    for (uint32_t t0 = tb; t0 < te; t0 += G::SP) {
        __syncthreads();  // the previous step's readers are done (and the tables are filled)
        if (a.cw)
            gm_stage_wc<F, SP>(a, n0, t0, threadIdx.x, lds);
        else
            gm_stage_w<F, SP>(a, src, tab, n0, t0, threadIdx.x, lds);
        gm_stage_x<F, Sh::BM, SP>(a, m0, t0, threadIdx.x, lds);
        __syncthreads();
        const uint32_t nsp = te - t0 < G::SP ? te - t0 : G::SP;
        for (uint32_t sp = 0; sp < nsp; sp++) {
            GmOps<NI, MJ> o;
            gm_ops<F, NI, MJ, SP>(lds, w, lane, sp, o);
            GmI<F, NI, MJ> I;
#pragma unroll
            for (uint32_t h = 0; h < G::NH; h++)
#pragma unroll
                for (int j = 0; j < MJ; j++) {
                    const uint64_t b = gm_half<F>(o.B[j], lane, h);
#pragma unroll
                    for (int i = 0; i < NI; i++) {
                        const gm_i32x4 z = {0, 0, 0, 0};
                        const gm_i32x4 r = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)o.A[i], (long)b, z, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; e++) I.v[h][i][j][e] = r[e];
                    }
                }
            gm_epi<F, NI, MJ, SP>(lds, w, lane, sp, I, acc);
        }
        if constexpr (G::AFF) {
            typedef float gm_f32x4 __attribute__((ext_vector_type(4)));
            const uint32_t nk = nsp * G::NH;
            for (uint32_t q = 0; 4u * q < nk; q++) {
                float A[NI], B[MJ];
                gm_offsets_ops<F, NI, MJ, SP>(lds, w, lane, q, nk, A, B);
#pragma unroll
                for (int i = 0; i < NI; i++)
#pragma unroll
                    for (int j = 0; j < MJ; j++) {
                        gm_f32x4 c = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                        c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[i], B[j], c, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 4; e++) acc[i][j][e] = c[e];
                    }
            }
        }
    }
    gm_store<NI, MJ>(a, n0, m0, ks, w, lane, acc);
}

// The per-call weight rewrite (one item per thread).
template <int F>
__global__ __launch_bounds__(WG) void k_gemm_rewrite(GmArgs a, uint32_t *cw, float *cs, float *co) {
    using TS = TabSpec<F>;
    __shared__ uint64_t t8[TS::n8 > 0 ? TS::n8 : 1];
    __shared__ uint32_t t4[TS::n4 > 0 ? TS::n4 : 1];
    if constexpr (TS::n8 + TS::n4 > 0) {
        gv_fill_tables<F>(t8, t4, threadIdx.x);
        __syncthreads();
    }
    const Tab tab{t8, t4, nullptr, nullptr, 0xFFFFFFFFu, 1u};
    const GmSrc src{a.wbase, a.wlast};
    using G = GmFmt<F>;
    constexpr uint32_t GR = (uint32_t)WG / 8u;  // groups (rows) per workgroup
    GmSpan o;
    uint32_t n = 0u, t = 0u;
    const bool live =
        gm_rewrite_span<F>(a, src, tab, (uint64_t)blockIdx.x * WG + threadIdx.x, cw, &n, &t, o);
    // The workgroup's groups are rows n0 .. n0 + GR - 1 of one span octet q
    // unless they pass the last row: then its scales and offsets go through
    // LDS, so that consecutive threads store consecutive rows of one span
    // (whole 128-byte runs instead of words N apart).
    const uint64_t g80 = (uint64_t)blockIdx.x * GR;
    const uint32_t n0 = (uint32_t)(g80 % a.rows), q = (uint32_t)(g80 / a.rows);
    if (n0 + GR <= a.rows) {
        __shared__ float tw[G::NH][8][GR + 1], to[G::AFF ? G::NH : 1][8][GR + 1];
        const uint32_t j = threadIdx.x / 8u, sp = threadIdx.x % 8u;  // this thread's row and span in the tile
#pragma unroll
        for (uint32_t h = 0; h < G::NH; h++) {
            tw[h][sp][j] = live ? o.ws[h] : 0.0f;
            if constexpr (G::AFF) to[h][sp][j] = live ? o.ow[h] : 0.0f;
        }
        __syncthreads();
        const uint32_t sj = threadIdx.x % GR, ss = threadIdx.x / GR;  // store: row sj of span ss
        const uint32_t ts = 8u * q + ss;
        if (ts < a.kspans) {
#pragma unroll
            for (uint32_t h = 0; h < G::NH; h++) {
                cs[((uint64_t)ts * G::NH + h) * a.ldy + n0 + sj] = tw[h][ss][sj];
                if constexpr (G::AFF) co[((uint64_t)ts * G::NH + h) * a.ldy + n0 + sj] = to[h][ss][sj];
            }
        }
    } else if (live) {
#pragma unroll
        for (uint32_t h = 0; h < G::NH; h++) {
            cs[((uint64_t)t * G::NH + h) * a.ldy + n] = o.ws[h];
            if constexpr (G::AFF) co[((uint64_t)t * G::NH + h) * a.ldy + n] = o.ow[h];
        }
    }
}

// The K splits' partial outputs summed in split order: y[i] = ((p0 + p1) + p2) ...
template <int U>
__global__ __launch_bounds__(WG) void k_gemm_sum(const float *part, float *y, uint64_t n, uint32_t nsplit) {
    for (uint64_t i = (uint64_t)blockIdx.x * WG + threadIdx.x; i < n; i += (uint64_t)gridDim.x * WG) {
        float v = part[i];
        for (uint32_t s = 1; s < nsplit; s++) v = v + part[(uint64_t)s * n + i];
        y[i] = v;
    }
}

// ------------------------------------------------------------------ host side

// Plan of a call: (1) when the tiles are fewer than two per compute unit and
// K is long (8 steps or more), K is cut into nsplit ranges of sps steps (at
// least 4 each) so that about two workgroups per compute unit run (three
// with enough 64-row tiles, (3)); the
// partial outputs (nsplit * M * N binary32 values, at most 2 GiB) go to the
// workspace and are summed in split order.  (2) With more than 256
// activation rows (5 or more activation tiles per weight tile) the weight is
// rewritten once into the workspace (codes, scales, offsets) and the tiles
// copy it, instead of each tile rewriting it (measured up to +23% from 384
// rows, 1 to 15% slower at 144 to 256 rows: the copy is about twice the
// packed bytes).  The results are the same bits either way for (2).  (3) With
// 64-row tiles, more than two per compute unit, K steps hold 4 spans
// instead of 8 (measured 9-25% faster between two and three, 5-23% above;
// at exactly two, one pass of 8-span workgroups, up to 45% slower); with
// five eighths to two such tiles per compute unit,
// K is split for three workgroups per compute unit, also in 4-span steps
// (measured up to +46%; at half a tile per compute unit and below it lost
// up to 32%).  The plan depends only on N, K, M and the compute-unit count.
struct GmPlan {
    uint32_t nsplit, sps;
    bool rewrite_once;  // the weight rewritten once per call (into the workspace)
    uint32_t sp;        // spans per K step (4 or 8)
};

// The plan without a workspace: no K split (and then 8-span steps where the
// 4-span ones came with a split), the weight rewritten per tile.
inline GmPlan gm_plan_plain(const GmPlan &p, uint64_t K) {
    const uint32_t sp = p.nsplit > 1 ? GM_SP : p.sp;
    return GmPlan{1u, (uint32_t)((K / 32 + sp - 1) / sp), false, sp};
}

// Activation rows above which format f's weight is rewritten once per call
// (into the workspace) instead of per tile.  At 320 and 384 rows
// ([14336, 4096] and [4096, 14336]) the per-tile rewrite measured 6-13%
// faster for q4_k, q2_k and tq2_0 (and 0-9% for q8_k), while q4_0, q4_1,
// q5_0, q5_k, iq2_xxs and iq3_s lost 5-21% without the once-per-call copy.
NQ_HD constexpr uint64_t gm_rewrite_m(int f) {
    return (f == Q4_K || f == Q2_K || f == TQ2_0 || f == Q8_K) ? 384u : GM_REWRITE_ONCE_M;
}

inline GmPlan gm_plan(int f, uint64_t N, uint64_t K, uint64_t M, uint32_t cus) {
    const uint64_t bm = gm_bm(M), tiles = (N + GM_BN - 1) / GM_BN * ((M + bm - 1) / bm);
    const uint64_t c = cus ? cus : 1u;
    const uint32_t sp0 = bm == 64u && tiles > 2ull * c ? 4u : GM_SP;
    const GmPlan p{1u, (uint32_t)((K / 32 + sp0 - 1) / sp0), M > gm_rewrite_m(f), sp0};
    if (tiles >= 2ull * c) return p;
    // K split; with 64-row tiles, five eighths to two per compute unit, into
    // 4-span steps and enough ranges for three workgroups per compute unit,
    // unless 8-span steps (two workgroups per compute unit, the split count
    // rounded down) fill at least nine tenths of their slots while the
    // 4-span split would spill a tail past its three per compute unit: at
    // 0.625 tiles per compute unit (3 splits: 480 of 512 slots against 800
    // workgroups for 768) that measured 1-10% faster on five formats, while
    // at 0.75 (2 splits: 384 of 512) it lost 14-24%.
    bool mid = bm == 64u && 8u * tiles >= 5u * c;
    if (mid) {
        const uint64_t s8 = 2u * c / tiles, s4 = (3u * c + tiles - 1) / tiles;
        if (s8 >= 2u && 10u * s8 * tiles >= 18u * c && s4 * tiles > 3u * c) mid = false;
    }
    const uint32_t sp = mid ? 4u : GM_SP;
    const uint64_t steps = (K / 32 + sp - 1) / sp, target = (mid ? 3ull : 2ull) * c;
    if (steps < 8) return p;
    // 64-row tiles in 8-span steps: two workgroups per compute unit fit, so
    // the split count rounds down (the grid stays within one pass of them;
    // rounding up left a tail pass, measured 7-36% slower); the other shapes
    // fit three and round up
    uint64_t S = bm == 64u && !mid ? target / tiles : (target + tiles - 1) / tiles;
    if (S > steps / 4) S = steps / 4;
    if (S < 2) return p;
    const uint64_t sps = (steps + S - 1) / S;
    S = (steps + sps - 1) / sps;
    if (S < 2 || S * M * N * 4 > (1ull << 31)) return p;
    return GmPlan{(uint32_t)S, (uint32_t)sps, p.rewrite_once, sp};
}

// Workspace layout: the split partials (nsplit * M * N binary32), then the
// rewritten weight: codes (N * K bytes), scales and, for the affine formats,
// offsets (K / 32 * NH * N binary32 each); every part 256-byte aligned.
struct GmWsLayout {
    uint64_t part, codes, scales, offsets, total;
};

inline GmWsLayout gm_ws_layout(int f, const GmPlan &p, uint64_t N, uint64_t K, uint64_t M) {
    auto up = [](uint64_t x) { return (x + 255) / 256 * 256; };
    GmWsLayout l{0, 0, 0, 0, 0};
    uint64_t at = p.nsplit > 1 ? up((uint64_t)p.nsplit * M * N * 4) : 0;
    if (p.rewrite_once) {
        const uint64_t sc = up(K / 32 * (gm_u16(f) ? 2u : 1u) * N * 4);
        l.codes = at;
        l.scales = l.codes + up(N * K);
        l.offsets = l.scales + sc;
        at = l.offsets + (gm_aff(f) ? sc : 0);
    }
    l.total = at;
    return l;
}

// One launch: weight rows r0 .. r0+rows-1, activation rows m0 .. m0+mrows-1,
// outputs into `out` ([M, N], or the [nsplit, M, N] partials); `canon` the
// workspace when the weight is rewritten once (null otherwise).
template <int F>
GmArgs gm_args(const GvLaunch &L, uint64_t r0, uint64_t rows, uint64_t m0, uint64_t mrows, const GmPlan &p,
               float *out, uint8_t *canon = nullptr, const GmWsLayout *wl = nullptr) {
    constexpr uint64_t S = (uint64_t)block_bytes(F);
    const uint64_t nbr = L.K / (uint64_t)block_values(F), row_bytes = nbr * S;
    const uint8_t *start = L.w + r0 * row_bytes;
    GmArgs a;
    a.wbase = (const uint32_t *)((uintptr_t)start & ~(uintptr_t)3);
    a.wmis = (uint32_t)((uintptr_t)start & 3u);
    a.wlast = (uint32_t)((a.wmis + rows * row_bytes - 1) / 4);
    a.xq = (const uint32_t *)L.xq + m0 * (L.K / 32 * 9);
    a.y = out + m0 * L.N + r0;
    a.rows = (uint32_t)rows;
    a.row_bytes = (uint32_t)row_bytes;
    a.kspans = (uint32_t)(L.K / 32);
    a.xrow = (uint32_t)(L.K / 32 * 9);
    a.ldy = (uint32_t)L.N;
    a.M = (uint32_t)mrows;
    a.bm = gm_bm(L.M);
    a.mt = (uint32_t)((mrows + a.bm - 1) / a.bm);
    a.nsplit = p.nsplit;
    a.sps = p.sps;
    a.ysplit = L.M * L.N;
    a.cw = canon ? (const uint32_t *)(canon + wl->codes + r0 * L.K) : nullptr;
    a.cs = canon ? (const float *)(canon + wl->scales) + r0 : nullptr;
    a.co = canon ? (const float *)(canon + wl->offsets) + r0 : nullptr;
    const uint64_t grid = (rows + GM_BN - 1) / GM_BN * a.mt * p.nsplit;
    a.xq8 = (uint32_t)(grid / 8);
    a.xr8 = (uint32_t)(grid % 8);
    return a;
}

inline uint32_t gm_grid(const GmArgs &a) { return 8u * a.xq8 + a.xr8; }

// Weight rows per launch: byte offsets fit 32 bits, and so do the byte
// offsets of the rewritten codes (K per row), whole tiles when more than
// one, and at most 2^24 rows (the grid stays below 2^31).
template <int F>
uint64_t gm_max_rows(const GvLaunch &L) {
    uint64_t r = gv_max_rows<F>(L);
    const uint64_t by_codes = (1ull << 32) / L.K;
    if (r > by_codes) r = by_codes;
    if (r > (1ull << 24)) r = 1ull << 24;
    return r >= GM_BN ? r / GM_BN * GM_BN : r;
}

// The call's launches; `ws` (ws_bytes) is the caller's workspace: with at
// least the plan's workspace (gm_ws_layout), K is split and the weight
// rewritten once as planned, else neither.
template <int F>
int launch_gemm_mfma(const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t stream) {
    const uint64_t max_rows = gm_max_rows<F>(L);
    GmPlan p = gm_plan(F, L.N, L.K, L.M, L.cus);
    // (the rewritten scales, K / 32 * NH * N words, take 32-bit byte offsets)
    const bool use = ws != nullptr && ws_bytes >= gm_ws_layout(F, p, L.N, L.K, L.M).total &&
                     (p.nsplit > 1 || p.rewrite_once) && (L.K / 32u) * 2u * L.N * 4u < (1ull << 32);
    if (!use) p = gm_plan_plain(p, L.K);
    const GmWsLayout wl = gm_ws_layout(F, p, L.N, L.K, L.M);
    const bool split = p.nsplit > 1;
    float *out = split ? (float *)ws : L.y;
    uint8_t *canon = p.rewrite_once ? (uint8_t *)ws : nullptr;
    if (canon) {
        for (uint64_t r0 = 0; r0 < L.N;) {
            const uint64_t rows = L.N - r0 < max_rows ? L.N - r0 : max_rows;
            const GmArgs a = gm_args<F>(L, r0, rows, 0, 1, p, out, canon, &wl);
            const uint64_t blocks = (gm_rewrite_items(a.rows, a.kspans) + WG - 1) / WG;
            hipLaunchKernelGGL((k_gemm_rewrite<F>), dim3((uint32_t)blocks), dim3(WG), 0, stream, a,
                               (uint32_t *)(canon + wl.codes + r0 * L.K), (float *)(canon + wl.scales) + r0,
                               (float *)(canon + wl.offsets) + r0);
            if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
            r0 += rows;
        }
    }
    const uint64_t max_mrows = gm_max_mrows(L.K);
    for (uint64_t m0 = 0; m0 < L.M; m0 += max_mrows) {
        const uint64_t mrows = L.M - m0 < max_mrows ? L.M - m0 : max_mrows;
        for (uint64_t r0 = 0; r0 < L.N;) {
            const uint64_t rows = L.N - r0 < max_rows ? L.N - r0 : max_rows;
            const GmArgs a = gm_args<F>(L, r0, rows, m0, mrows, p, out, canon, &wl);
            if (a.bm == 64u && p.sp == 4u)
                hipLaunchKernelGGL((k_gemm<F, 4, 2, 4>), dim3(gm_grid(a)), dim3(WG), 0, stream, a);
            else if (a.bm == 64u)
                hipLaunchKernelGGL((k_gemm<F, 4, 2, 8>), dim3(gm_grid(a)), dim3(WG), 0, stream, a);
            else if (a.bm == 32u)
                hipLaunchKernelGGL((k_gemm<F, 4, 1, 8>), dim3(gm_grid(a)), dim3(WG), 0, stream, a);
            else
                hipLaunchKernelGGL((k_gemm<F, 2, 1, 8>), dim3(gm_grid(a)), dim3(WG), 0, stream, a);
            if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
            r0 += rows;
        }
    }
    if (split) {
        const uint64_t n = L.M * L.N, blocks = (n + WG - 1) / WG;
        hipLaunchKernelGGL((k_gemm_sum<0>), dim3((uint32_t)(blocks < 8192 ? blocks : 8192)), dim3(WG), 0, stream,
                           (const float *)ws, L.y, n, p.nsplit);
        if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
    }
    return 0;
}

// Products with more than 8 activation rows on the matrix cores (formats
// with a span rewrite; the others, and fewer rows, go through the
// single-row kernel).
template <int F>
int launch_gemm_f(const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t stream) {
    if constexpr (GmFmt<F>::OK)
        return launch_gemm_mfma<F>(L, ws, ws_bytes, stream);
    else
        return 2;  // NQ_ERR_UNKNOWN_FORMAT
}

}  // namespace nq
