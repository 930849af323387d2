// nq_fp8row.h -- row-scaled FP8 decode: fp8_e4m3fn_row_bf16 / _fp16.
//
// NInfer "tensor-formats" page, section 3.3: a rank-two [N, K] matrix of
// E4M3FN code words with one bfloat16 (section 3.1) or binary16 multiplier
// per row; each value is the binary32 product code * scale, then converted
// once to the output type like every other decode here.  Bytes: the N*K codes
// row-major, then the N scale words (little-endian 16-bit) in row order.
//
// Launch shape: one thread per 16 consecutive values of the flat output, 256
// threads per workgroup, one workgroup per 4096 values.  A thread reads its
// 16 codes as one 16-byte window (any payload alignment), the scale word of
// each row its values touch, and stores two 8-value units (one 16-byte
// store each for bf16/f16 outputs).  A launch covers at most 2^30 values; the
// host splits larger matrices into such chunks.
#pragma once

#include "nq_kernel.h"

namespace nq {

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
// value where the following row starts.
NQ_HD uint32_t f8_row(const F8Args &a, uint32_t e, uint64_t *next) {
    const uint64_t col = (uint64_t)a.col0 + e;
    uint64_t r;
    if (a.K <= 0xFFFFFFFFull && col <= 0xFFFFFFFFull)
        r = (uint32_t)col / (uint32_t)a.K;
    else
        r = col / a.K;
    *next = (r + 1) * a.K - a.col0;
    return (uint32_t)r;
}

// The work of thread i: values 16i .. 16i+15 of the launch (those below n).
template <int SK, int OT, bool VEC, class Src>
NQ_HD void fp8row_thread(const Src &csrc, const Src &ssrc, const F8Args &a, uint32_t i) {
    const uint32_t e = 16u * i;
    if (e >= a.n) return;
    const bool full = a.n - e >= 16u;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (full) {
        window<4>(csrc, a.cmis + e, w);
    } else {
        for (uint32_t j = 0; j < a.n - e; j++) w[j >> 2] |= u8_at(csrc, a.cmis + e + j) << (8u * (j & 3u));
    }
    uint64_t next;
    uint32_t r = f8_row(a, e, &next);
    float s = row_scale<SK>(u16_at(ssrc, a.smis + 2u * r));
    float y[16];
#pragma unroll
    for (uint32_t j = 0; j < 16; j++) {
        if ((uint64_t)e + j == next && e + j < a.n) {  // a row starts inside this thread's values
            r++;
            next += a.K;
            s = row_scale<SK>(u16_at(ssrc, a.smis + 2u * r));
        }
        y[j] = M(e4m3fn_exact(bytek(w[j >> 2], j & 3u)), s);
    }
    if (full) {
        float lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            lo[j] = y[j];
            hi[j] = y[8 + j];
        }
        store8<OT, VEC>(a.out, 2u * i, lo);
        store8<OT, VEC>(a.out, 2u * i + 1u, hi);
    } else {
        for (uint32_t j = 0; j < a.n - e; j++) store1<OT>(a.out, (uint64_t)e + j, y[j]);
    }
}

template <int SK, int OT, bool VEC>
__global__ __launch_bounds__(WG) void k_fp8_row(F8Args a) {
    fp8row_thread<SK, OT, VEC>(DevSrc{a.cbase, a.clast}, DevSrc{a.sbase, a.slast}, a,
                               blockIdx.x * (uint32_t)WG + threadIdx.x);
}

// Host side: one matrix, split into launches of at most 2^30 values.
struct F8Launch {
    const uint8_t *payload;  // device
    uint64_t N, K;
    void *out;               // device
};

constexpr uint64_t F8_CHUNK = 1ull << 30;

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
    *grid = (uint32_t)((n + 16u * WG - 1) / (16u * WG));
    return a;
}

int launch_fp8_row(int scale_kind, int ot, const F8Launch &L, hipStream_t s);

}  // namespace nq
