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
// and activation rows m < M <= 8, in binary32 with fused multiply-adds.  A
// wave owns RW weight rows; its 64 lanes take the row's 8-value units in
// turn (lane l: units l, l+64, ...), decode each unit exactly as the decode
// kernels do, and keep one FP32 partial per (row, activation row); the
// partials then meet in a fixed cross-lane tree, so every run gives the same
// bits.  Lanes that handle the same unit for several rows read the unit's
// activation codes once.
#pragma once

#include "nq_gqenc.h"

namespace nq {

constexpr int GV_MAX_M = 8;

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

// Phase 2 of a lane (after amax and the failure flag are combined over the
// block's lanes): the block's d word, the lane's codes (zero when the block
// fails) and status bits 1 and 2.
template <int VPL>
NQ_HD uint32_t q81_encode(float amax, bool bad, const float (&v)[VPL], uint32_t *d16, int8_t (&q)[VPL]) {
    uint32_t st = bad ? 1u : gq_encode<3, VPL>(amax, v, d16, q);
    if (st) {
        *d16 = 0u;
#pragma unroll
        for (int k = 0; k < VPL; k++) q[k] = 0;
    }
    return st;
}

// Phase 3 (after the code sums are combined): lane j of block b stores its
// codes; lane 0 stores the d and sum words.  Returns the block's status bits
// (lane 0 reports them).
template <int VPL>
NQ_HD uint32_t q81_store(const Q81Args &a, uint32_t b, uint32_t j, const int8_t (&q)[VPL], uint32_t d16, int sum,
                     uint32_t st) {
    const uint32_t s16 = gq_f32_to_f16(f16(d16) * (float)sum);  // exact product, one rounding
    if ((s16 & 0x7C00u) == 0x7C00u) st |= 4u;
    uint32_t *blk = a.blocks + (uint64_t)b * 9u;
#pragma unroll
    for (int d = 0; d < VPL / 4; d++) {
        uint32_t w = 0u;
#pragma unroll
        for (int k = 0; k < 4; k++) w |= (uint32_t)(uint8_t)q[4 * d + k] << (8 * k);
        blk[1u + j * (uint32_t)(VPL / 4) + (uint32_t)d] = w;
    }
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
    float amax = 0.0f;
    bool bad = false;
    if (live) {
        gq_load<IN, VECIN>(GqDevSrc{a.x}, (uint64_t)b * 32u + j * (uint32_t)VPL, (uint32_t)VPL, v, &amax, &bad);
    } else {
#pragma unroll
        for (int k = 0; k < VPL; k++) v[k] = 0.0f;
    }
    // every lane of the wave takes part in the exchanges
#pragma unroll
    for (uint32_t off = LPB / 2; off >= 1; off >>= 1) {
        const float o = __shfl_xor(amax, (int)off, 64);
        amax = o > amax ? o : amax;
        bad |= __shfl_xor((int)bad, (int)off, 64) != 0;
    }
    int8_t q[VPL];
    uint32_t d16 = 0u;
    const uint32_t st = q81_encode<VPL>(amax, bad, v, &d16, q);
    int sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; k++) sum += q[k];
#pragma unroll
    for (uint32_t off = LPB / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, (int)off, 64);
    if (live) {
        const uint32_t bits = q81_store<VPL>(a, b, j, q, d16, sum, st);
        if (bits && j == 0u) atomicOr(a.status, bits);
    }
}

// ------------------------------------------------------------------ product

struct GvArgs {
    const uint32_t *wbase;  // weight bytes of this launch's first row, aligned down to 4 bytes
    uint32_t wmis;          // that row's start - wbase (0..3)
    uint32_t wlast;         // last dword holding weight bytes of this launch, from wbase
    const uint32_t *xq;     // q8_1 activation blocks; activation row m starts at dword m * xrow
    float *y;               // output of this launch's first weight row; activation row m at m * ldy
    uint32_t rows;          // weight rows in this launch
    uint32_t row_bytes;     // bytes per weight row, K / B * S
    uint32_t K;             // values per row
    uint32_t xrow;          // dwords per activation row, K / 32 * 9
    uint32_t ldy;           // N
    uint32_t M;             // activation rows, 1 .. MT
};

// Sum over the 64 lanes of a wave in a fixed butterfly order; every lane ends
// with the same value.
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// q8_1 code j (0..7) of the two dwords c.
NQ_HD float q8_code(const uint32_t (&c)[2], int j) {
    return (float)(int8_t)(c[j >> 2] >> (8 * (j & 3)));
}

// One lane's partial sums for the RW weight rows r0.. of its wave: the row's
// units lane, lane + 64, ..., each decoded to 8 binary32 weights and
// multiplied with the unit's 8 activation codes (FMA chain), then scaled by
// the activation block's d and added to the partial.
template <int F, int MT, int RW, class Src>
NQ_HD void gv_lane(const Src &src, const Tab &tab, const GvArgs &a, uint32_t r0, uint32_t lane,
                   float (&acc)[RW][MT]) {
    constexpr uint32_t UPB = (uint32_t)block_values(F) / 8u, S = (uint32_t)block_bytes(F);
#pragma unroll
    for (int rr = 0; rr < RW; rr++)
#pragma unroll
        for (int m = 0; m < MT; m++) acc[rr][m] = 0.0f;
    const uint32_t U = a.K >> 3;
    for (uint32_t u = lane; u < U; u += 64u) {
        const uint32_t xo = (u >> 2) * 9u, co = 1u + 2u * (u & 3u);
        float xd[MT];
        uint32_t xc[MT][2];
#pragma unroll
        for (int m = 0; m < MT; m++) {
            if (m < (int)a.M) {
                const uint32_t *p = a.xq + (uint64_t)m * a.xrow + xo;
                xd[m] = f16(p[0] & 0xFFFFu);
                xc[m][0] = p[co];
                xc[m][1] = p[co + 1u];
            }
        }
#pragma unroll
        for (int rr = 0; rr < RW; rr++) {
            const uint32_t r = r0 + (uint32_t)rr;
            if (r >= a.rows) continue;
            float w[8];
            decode_unit<F>(src, a.wmis + r * a.row_bytes + (u / UPB) * S, u % UPB, tab, w);
#pragma unroll
            for (int m = 0; m < MT; m++) {
                if (m >= (int)a.M) continue;
                float t = w[0] * q8_code(xc[m], 0);
#pragma unroll
                for (int j = 1; j < 8; j++) t = __builtin_fmaf(w[j], q8_code(xc[m], j), t);
                acc[rr][m] = __builtin_fmaf(t, xd[m], acc[rr][m]);
            }
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

// Workgroup g (and g + grid, ...) takes weight rows 4*RW*g .. 4*RW*g + 4*RW - 1,
// wave w of it rows 4*RW*g + RW*w ...
template <int F, int MT, int RW>
__global__ __launch_bounds__(WG) void k_gemv_unit(GvArgs a) {
    using TS = TabSpec<F>;
    __shared__ uint64_t t8[TS::n8 > 0 ? TS::n8 : 1];
    __shared__ uint32_t t4[TS::n4 > 0 ? TS::n4 : 1];
    if constexpr (TS::n8 + TS::n4 > 0) {
        gv_fill_tables<F>(t8, t4, threadIdx.x);
        __syncthreads();
    }
    const Tab tab{t8, t4, nullptr, nullptr, 0xFFFFFFFFu, 1u};
    const DevSrc src{a.wbase, a.wlast};
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    for (uint32_t g = blockIdx.x; g * (4u * RW) < a.rows; g += gridDim.x) {
        const uint32_t r0 = (g * 4u + wave) * (uint32_t)RW;
        float acc[RW][MT];
        gv_lane<F, MT, RW>(src, tab, a, r0, lane, acc);
#pragma unroll
        for (int rr = 0; rr < RW; rr++) {
            const uint32_t r = r0 + (uint32_t)rr;
#pragma unroll
            for (int m = 0; m < MT; m++) {
                const float s = wave_sum(acc[rr][m]);
                if (lane == 0u && r < a.rows && m < (int)a.M) a.y[(uint64_t)m * a.ldy + r] = s;
            }
        }
    }
}

// Arguments and grid size of the launch for rows r0 .. r0 + rows - 1.
// Host description of one product call.
struct GvLaunch {
    const uint8_t *w;   // device weight payload [N, K]
    uint64_t N, K, M;
    const uint8_t *xq;  // device q8_1 activation blocks [M, K / 32]
    float *y;           // device output [M, N]
    uint32_t resident;  // workgroups the device holds at once
};

struct Q81Launch {
    const void *x;
    uint64_t nblocks;
    uint32_t *blocks;
    uint32_t *status;
};

// Rows per wave: two when at most two activation rows (the unit's codes are
// shared by both rows), else one (register budget).
template <int MT>
constexpr int gv_rw() {
    return MT <= 2 ? 2 : 1;
}

template <int F, int MT>
GvArgs gv_args(const GvLaunch &L, uint64_t r0, uint64_t rows, uint32_t *grid) {
    constexpr int RW = gv_rw<MT>();
    constexpr bool TABLES = TabSpec<F>::n8 + TabSpec<F>::n4 > 0;
    const uint64_t row_bytes = L.K / (uint64_t)block_values(F) * (uint64_t)block_bytes(F);
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
    a.xrow = (uint32_t)(L.K / 32 * 9);
    a.ldy = (uint32_t)L.N;
    a.M = (uint32_t)L.M;
    uint64_t groups = (rows + 4u * RW - 1) / (4u * RW);
    // formats with codebooks fill them per workgroup: fewer workgroups, each looping
    if (TABLES && groups > L.resident) groups = L.resident;
    *grid = (uint32_t)groups;
    return a;
}

// Rows per launch: every weight byte offset of a launch fits 32 bits.
template <int F>
uint64_t gv_max_rows(const GvLaunch &L) {
    return 0xFFFFFFF0ull / (L.K / (uint64_t)block_values(F) * (uint64_t)block_bytes(F));
}

template <int F, int MT>
int launch_gemv_mt(const GvLaunch &L, hipStream_t stream) {
    const uint64_t max_rows = gv_max_rows<F>(L);
    for (uint64_t r0 = 0; r0 < L.N;) {
        const uint64_t rows = L.N - r0 < max_rows ? L.N - r0 : max_rows;
        uint32_t grid;
        const GvArgs a = gv_args<F, MT>(L, r0, rows, &grid);
        hipLaunchKernelGGL((k_gemv_unit<F, MT, gv_rw<MT>()>), dim3(grid), dim3(WG), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
        r0 += rows;
    }
    return 0;
}

template <int F>
int launch_gemv_f(const GvLaunch &L, hipStream_t s) {
    if (L.M <= 1) return launch_gemv_mt<F, 1>(L, s);
    if (L.M <= 2) return launch_gemv_mt<F, 2>(L, s);
    if (L.M <= 4) return launch_gemv_mt<F, 4>(L, s);
    return launch_gemv_mt<F, 8>(L, s);
}

}  // namespace nq
