// nq_fp8row.h -- row-scaled FP8 decode: fp8_e4m3fn_row_bf16 / _fp16.
//
// NInfer "tensor-formats" page, section 3.3: a rank-two [N, K] matrix of
// E4M3FN code words with one bfloat16 (section 3.1) or binary16 multiplier
// per row; each value is the binary32 product code * scale, then converted
// once to the output type like every other decode here.  Bytes: the N*K codes
// row-major, then the N scale words (little-endian 16-bit) in row order.
//
// Launch shape: units of 8 consecutive values, decoded in wave blocks of 128
// units (see k_fp8_row): one 1 KiB code load per wave, passed through the
// wave's own LDS so that each store instruction writes 64 consecutive units
// (1 KiB for bf16/f16), as in the block decoders.  A launch covers at most
// 2^30 values; the host splits larger matrices into such chunks.
#pragma once

#include "nq_kernel.h"

namespace nq {

constexpr uint64_t F8_CHUNK = 1ull << 30;  // values per launch at most

// One launch: values [E0, E0 + n) of the matrix.
struct F8Args {
    const uint32_t *cbase;  // codes from value E0, aligned down to 4 bytes
    const uint32_t *sbase;  // scale words from row E0 / K, aligned down to 4 bytes
    void *out;              // output value E0
    uint64_t K;             // row length
    uint32_t cmis, clast;   // code start - cbase (0..3); last dword holding chunk codes
    uint32_t smis, slast;   // scale start - sbase (0..3); last dword holding chunk scales
    uint32_t n;             // values in this launch (<= 2^30)
    uint64_t col0;          // column of value E0 (E0 mod K)
    uint32_t kmul, kshift;  // division by K <= 2^30 as a multiply-shift (div_magic)
};

// Exact E4M3FN value: the 7 magnitude bits placed at binary32 bits 26..20
// give 2^-120 times the value (a binary32 subnormal when the E4M3FN exponent
// is 0), so one exact multiplication by 2^120 finishes it; 0x7F/0xFF are NaN.
NQ_HD float e4m3fn_exact(uint32_t w) {
    const uint32_t mag = w & 0x7Fu;
    const float v = M(bits_f32(mag << 20), 0x1p120f);
    const uint32_t b = mag == 0x7Fu ? 0x7FC00000u : __builtin_bit_cast(uint32_t, v);
    return bits_f32(b | ((w & 0x80u) << 24));
}

template <int SK>
NQ_HD float row_scale(uint32_t w) {
    if constexpr (SK == 0)
        return bits_f32(w << 16);  // bfloat16: the word in the high half
    else
        return f16(w);
}

// Row of chunk value e relative to the chunk's first row, and the chunk
// value where the following row starts.  col = col0 + e < K + 2^30 (a launch
// holds at most 2^30 values and col0 < K): for K <= 2^30 it fits 31 bits, and
// for longer rows the quotient is 0 or 1, so no 64-bit division is needed.
NQ_HD uint32_t f8_row(const F8Args &a, uint32_t e, uint64_t *next) {
    const uint64_t col = a.col0 + e;
    uint32_t r;
    if (a.K <= F8_CHUNK)
        r = (uint32_t)(((uint64_t)(uint32_t)col * a.kmul) >> a.kshift);
    else
        r = col >= a.K ? 1u : 0u;
    *next = (uint64_t)(r + 1) * a.K - a.col0;
    return r;
}

// Row-scale words are read per unit (rows are long next to a unit, and the
// lanes of a wave mostly share one row, so these loads hit one cache line).
// With K >= 8 a unit touches at most two rows: values before the next row's
// start take the first row's scale, the rest the second's (loaded only then).
// Whether one of the 4 code bytes of x is a NaN word (magnitude 0x7F): with
// bit 7 forced on in every byte, such a byte is 0xFF, i.e. a zero byte of the
// complement, found by the usual borrow test (exact as a yes/no answer).
NQ_HD uint32_t f8_has_nan(uint32_t x) { return (~(x | 0x80808080u) - 0x01010101u) & 0x80808080u; }

// E4M3FN value of a code byte that is not a NaN word.
NQ_HD float e4m3fn_exact_finite(uint32_t c) {
    const float v = M(bits_f32((c & 0x7Fu) << 20), 0x1p120f);
    return bits_f32(__builtin_bit_cast(uint32_t, v) | ((c & 0x80u) << 24));
}

template <int SK, class Src>
NQ_HD void fp8row_values(const Src &ssrc, const F8Args &a, uint32_t u, const uint32_t (&w)[2], float (&y)[8]) {
    const uint32_t e = 8u * u;
    uint64_t next;
    const uint32_t r = f8_row(a, e, &next);
    const float s = row_scale<SK>(u16_at(ssrc, a.smis + 2u * r));
    const uint32_t split = next - e < 8u ? (uint32_t)(next - e) : 8u;  // first value of the next row
    if (split == 8u && (f8_has_nan(w[0]) | f8_has_nan(w[1])) == 0u) {  // one row, no NaN words
#pragma unroll
        for (uint32_t j = 0; j < 8; j++) y[j] = M(e4m3fn_exact_finite(bytek(w[j >> 2], j & 3u)), s);
        return;
    }
    float s2 = s;
    if (split < 8u && e + split < a.n) s2 = row_scale<SK>(u16_at(ssrc, a.smis + 2u * (r + 1u)));
#pragma unroll
    for (uint32_t j = 0; j < 8; j++) y[j] = M(e4m3fn_exact(bytek(w[j >> 2], j & 3u)), j < split ? s : s2);
}

// Rows shorter than a unit (K < 8): value by value, each with its own row.
template <int SK, int OT, class Src>
NQ_HD void fp8row_values_short_rows(const Src &csrc, const Src &ssrc, const F8Args &a, uint32_t u) {
    const uint32_t e = 8u * u;
#pragma unroll 1
    for (uint32_t j = 0; j < 8u && e + j < a.n; j++) {
        uint64_t next;
        const uint32_t r = f8_row(a, e + j, &next);
        const float s = row_scale<SK>(u16_at(ssrc, a.smis + 2u * r));
        store1<OT>(a.out, (uint64_t)e + j, M(e4m3fn_exact(u8_at(csrc, a.cmis + e + j)), s));
    }
}

// One unit read straight from global memory: a byte-shifted two-word window,
// or byte by byte for the last, partial unit.
template <int SK, int OT, bool VEC, class Src>
NQ_HD void fp8row_unit_direct(const Src &csrc, const Src &ssrc, const F8Args &a, uint32_t u) {
    const uint32_t e = 8u * u;
    if (e >= a.n) return;
    if (a.K < 8u) {
        fp8row_values_short_rows<SK, OT>(csrc, ssrc, a, u);
        return;
    }
    uint32_t w[2] = {0u, 0u};
    const bool full = a.n - e >= 8u;
    if (full) {
        window<2>(csrc, a.cmis + e, w);
    } else {
        for (uint32_t j = 0; e + j < a.n; j++) w[j >> 2] |= u8_at(csrc, a.cmis + e + j) << (8u * (j & 3u));
    }
    float y[8];
    fp8row_values<SK>(ssrc, a, u, w, y);
    if (full) {
        store8<OT, VEC>(a.out, u, y);
    } else {
        for (uint32_t j = 0; e + j < a.n; j++) store1<OT>(a.out, (uint64_t)e + j, y[j]);
    }
}

// Work split: a wave block is 128 units (1 KiB of codes).  Wave v of
// workgroup b takes wave blocks (4b + v) * F8_NB + k, k < F8_NB.  When the
// codes start on a 4-byte boundary and the block holds 128 whole units, lane
// l loads 16 consecutive code bytes (units 2l, 2l+1; one 1 KiB load per
// wave), the wave passes them through its own 1 KiB of LDS, and lane l then
// decodes units l and 64 + l, so each store instruction of the wave writes
// 64 consecutive units.  Other blocks decode unit by unit from global memory.
#ifndef NQ_F8_NB
#define NQ_F8_NB 2
#endif
constexpr int F8_NB = NQ_F8_NB;
constexpr uint32_t F8_WG_UNITS = 4u * 128u * F8_NB;

NQ_HD uint32_t f8_wave_block(uint32_t b, uint32_t wave, int k) { return (4u * b + wave) * F8_NB + (uint32_t)k; }

// Whether wave block q takes the fast path: codes on a 4-byte boundary, rows
// of at least 8 values, and 128 whole units in the block.
NQ_HD bool f8_fast_block(const F8Args &a, uint32_t q) {
    return a.cmis == 0 && a.K >= 8u && 128u * (q + 1) <= a.n / 8u;
}

// Phase 1 (fast blocks): lane l's 16 code bytes (units 2l, 2l+1).
template <class Src>
NQ_HD void fp8row_stage_load(const Src &csrc, uint32_t q, uint32_t lane, uint32_t (&w)[4]) {
    csrc.load_stream4(256u * q + 4u * lane, w);
}

// Phase 2 (fast blocks): lane l decodes units 128q + l and 128q + 64 + l from
// the wave's LDS words.
template <int SK, int OT, bool VEC, class Src>
NQ_HD void fp8row_wave_decode(const Src &ssrc, const F8Args &a, uint32_t q, uint32_t lane, const uint32_t *wbuf) {
#pragma unroll
    for (uint32_t h = 0; h < 2; h++) {
        const uint32_t v = 64u * h + lane;
        const uint32_t w[2] = {wbuf[2u * v], wbuf[2u * v + 1u]};
        float y[8];
        fp8row_values<SK>(ssrc, a, 128u * q + v, w, y);
        store8<OT, VEC>(a.out, 128u * q + v, y);
    }
}

// A workgroup whose wave blocks are all fast issues all of its code loads
// before its first LDS write; otherwise every unit is read directly.
template <int SK, int OT, bool VEC>
__global__ __launch_bounds__(WG) void k_fp8_row(F8Args a) {
    __shared__ __attribute__((aligned(16))) uint32_t buf[4][F8_NB][256];
    const uint32_t wave = threadIdx.x / 64u, lane = threadIdx.x % 64u;
    const DevSrc csrc{a.cbase, a.clast}, ssrc{a.sbase, a.slast};
    if (f8_fast_block(a, f8_wave_block(blockIdx.x, 3u, F8_NB - 1))) {  // the workgroup's last block
        uint32_t w[F8_NB][4];
#pragma unroll
        for (int k = 0; k < F8_NB; k++) fp8row_stage_load(csrc, f8_wave_block(blockIdx.x, wave, k), lane, w[k]);
#pragma unroll
        for (int k = 0; k < F8_NB; k++) {
            uint32_t *wb = buf[wave][k];
#pragma unroll
            for (int j = 0; j < 4; j++) wb[4u * lane + j] = w[k][j];
        }
        // the wave's LDS words are written and read by the same wave: a
        // wave-scope release/acquire around a wave barrier orders them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < F8_NB; k++)
            fp8row_wave_decode<SK, OT, VEC>(ssrc, a, f8_wave_block(blockIdx.x, wave, k), lane, buf[wave][k]);
    } else {
#pragma unroll
        for (int k = 0; k < F8_NB; k++) {
            const uint32_t q = f8_wave_block(blockIdx.x, wave, k);
            fp8row_unit_direct<SK, OT, VEC>(csrc, ssrc, a, 128u * q + lane);
            fp8row_unit_direct<SK, OT, VEC>(csrc, ssrc, a, 128u * q + 64u + lane);
        }
    }
}

// Host side: one matrix, split into launches of at most 2^30 values.
struct F8Launch {
    const uint8_t *payload;  // device
    uint64_t N, K;
    void *out;               // device
};

// Arguments of the launch covering values [E0, E0 + min(chunk, rest)).
template <int OT>
NQ_HD F8Args f8_chunk_args(const F8Launch &L, uint64_t E0, uint32_t *grid, uint64_t chunk = F8_CHUNK) {
    constexpr uint64_t OSZ = OT == 0 ? 4 : OT == 3 ? 8 : 2;
    const uint64_t total = L.N * L.K;
    const uint64_t n = total - E0 < chunk ? total - E0 : chunk;
    const uint64_t r0 = E0 / L.K, r1 = (E0 + n - 1) / L.K;
    const uint8_t *c = L.payload + E0;
    const uint8_t *sw = L.payload + total + 2 * r0;
    F8Args a;
    a.cbase = (const uint32_t *)((uintptr_t)c & ~(uintptr_t)3);
    a.cmis = (uint32_t)((uintptr_t)c & 3);
    a.clast = (uint32_t)((a.cmis + n - 1) >> 2);
    a.sbase = (const uint32_t *)((uintptr_t)sw & ~(uintptr_t)3);
    a.smis = (uint32_t)((uintptr_t)sw & 3);
    a.slast = (uint32_t)((a.smis + 2 * (r1 - r0 + 1) - 1) >> 2);
    a.out = (uint8_t *)L.out + E0 * OSZ;
    a.K = L.K;
    a.n = (uint32_t)n;
    a.col0 = E0 - r0 * L.K;
    a.kmul = 0;
    a.kshift = 0;
    if (L.K <= F8_CHUNK) div_magic(L.K, &a.kmul, &a.kshift);
    *grid = (uint32_t)((n + 8u * F8_WG_UNITS - 1) / (8u * F8_WG_UNITS));
    return a;
}

int launch_fp8_row(int scale_kind, int ot, const F8Launch &L, hipStream_t s);

}  // namespace nq
