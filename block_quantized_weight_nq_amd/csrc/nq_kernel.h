// nq_kernel.h -- the decode kernel template and its launcher.
//
// One kernel per (format, output type, tile size, vector store).  The output
// is cut into tiles of 256*UPT units (a unit is 8 consecutive outputs of one
// block), and each tile is one workgroup: it copies the tile's payload bytes
// into LDS with coalesced 16-byte loads, then decodes its units so that a
// wave's 64 lanes cover 64 consecutive units: one contiguous 1 KiB
// (bf16/f16) or 2 KiB (f32) run per store instruction.  A tile whose staging
// would pass the payload's end is decoded straight from global memory.  IQ
// formats copy their codebook to LDS in every workgroup; "nvfp4" fills a
// 1024-entry table of its correctly rounded quotients (128 scale magnitudes x
// 8 code magnitudes; signs are applied as bit flips).
#pragma once

#include "iq_grids.h"
#include "nq_decode.h"

// Tuning knobs (compile-time; the defaults are the measured best on MI355X):
//   NQ_NTL        1: load_stream4 (the row-scaled FP8 and product kernels'
//                 streaming loads) is non-temporal
//   NQ_STAGE_NT   the decode's staging loads: -1 (default) by launch size and
//                 format (stage_nt), 0 ordinary, 1 non-temporal for every launch
//   NQ_STAGE_NT_UNITS  launches below this many units stage non-temporally
//   NQ_UPT        units (8 outputs) per thread per tile for every launch
//                 (default: chosen per launch from its size, see choose_upt)
//   NQ_UPT_LONG   tile size of long launches for every format (default: per
//                 format, upt_long)
//   NQ_RESIDENT_PER_CU  workgroups a compute unit holds at once, the scale of
//                 the per-launch tile-size choice
//   NQ_NT_STORE   non-temporal output stores: 0 never, 1 always, 2 16-bit outputs only
#ifndef NQ_NTL
#define NQ_NTL 1
#endif
#ifndef NQ_STAGE_NT
#define NQ_STAGE_NT -1
#endif
#ifndef NQ_RESIDENT_PER_CU
#define NQ_RESIDENT_PER_CU 8
#endif

namespace nq {

typedef uint32_t u32x2a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// Payload source: dword loads from a 4-byte-aligned base; `last` is the index
// of the last dword that holds payload bytes (loads never go past it).
struct DevSrc {
    const uint32_t *base;
    uint32_t last;
    template <int N>
    NQ_HD void load(uint32_t i, uint32_t (&r)[N]) const {
        const uint32_t *p = base + i;
        if constexpr (N == 1) {
            r[0] = p[0];
        } else if constexpr (N == 2) {
            const u32x2a4 v = *(const u32x2a4 *)p;
            r[0] = v.x;
            r[1] = v.y;
        } else if constexpr (N == 3) {
            const u32x2a4 v = *(const u32x2a4 *)p;
            r[0] = v.x;
            r[1] = v.y;
            r[2] = p[2];
        } else {
            const u32x4a4 v = *(const u32x4a4 *)p;
            r[0] = v.x;
            r[1] = v.y;
            r[2] = v.z;
            r[3] = v.w;
        }
    }
    NQ_HD uint32_t dw(uint32_t i) const { return base[i]; }
    // the extra dword of a window, clamped to the last payload dword
    NQ_HD uint32_t dwx(uint32_t i) const { return base[i < last ? i : last]; }
    // 16 bytes, non-temporal when NT.
    template <bool NT>
    NQ_HD void load4(uint32_t i, uint32_t (&r)[4]) const {
        u32x4a4 v;
#if defined(__HIP_DEVICE_COMPILE__)
        if constexpr (NT)
            v = __builtin_nontemporal_load((const u32x4a4 *)(base + i));
        else
#endif
            v = *(const u32x4a4 *)(base + i);
        r[0] = v.x;
        r[1] = v.y;
        r[2] = v.z;
        r[3] = v.w;
    }
    // 16 bytes that are read once (non-temporal when NQ_NTL).
    NQ_HD void load_stream4(uint32_t i, uint32_t (&r)[4]) const { load4<NQ_NTL != 0>(i, r); }
};

// Lookup tables (LDS in the kernels, host arrays in the emulator).
struct Tab {
    const uint64_t *t8;
    const uint32_t *t4;
    const float *nvq;        // "nvfp4": quotients by the divisor of the tile's first unit
    const float *nvd;        // "nvfp4": divisors of the groups the tile reaches, from that one on
    uint32_t nv_bound;       // "nvfp4": first unit (chunk-relative) past that divisor's group
    uint32_t nv_gu;          // "nvfp4": units per divisor group, capped at 2^31 - 1
    uint32_t nv_dsign;       // "nvfp4": sign bit of the table's divisor in bit 7 of every byte
    NQ_HD uint64_t iq2xxs(uint32_t r) const { return t8[r]; }
    NQ_HD uint64_t iq2xs(uint32_t r) const { return t8[r]; }
    NQ_HD uint64_t iq2s(uint32_t r) const { return t8[r]; }
    NQ_HD uint64_t iq1s(uint32_t r) const { return t8[r]; }
    NQ_HD uint32_t iq3xxs(uint32_t r) const { return t4[r]; }
    NQ_HD uint32_t iq3s(uint32_t r) const { return t4[r]; }
    NQ_HD float nv(uint32_t k) const { return nvq[k]; }
    // "nvfp4": table word at byte offset b (b = 4 * entry)
    NQ_HD uint32_t nvb(uint32_t b) const { return *(const uint32_t *)((const char *)nvq + b); }
};

// Table sizes per format.
template <int F>
struct TabSpec {
    static constexpr int n8 = F == IQ2_XXS ? 256 : F == IQ2_XS ? 512 : F == IQ2_S ? 1024
                            : (F == IQ1_S || F == IQ1_M) ? 2048 : 0;
    static constexpr int n4 = F == IQ3_XXS ? 256 : F == IQ3_S ? 512 : 0;
    static constexpr int nf = F == NVFP4_DIV ? 1024 : 0;
    // divisors a tile can reach: a group is at least one row of 64 values
    // (8 units), a tile at most 16 * 256 units
    static constexpr int nd = F == NVFP4_DIV ? 1 + 16 * 256 / 8 : 0;
    NQ_HD static const uint64_t *src8() {
        return F == IQ2_XXS ? NQ_GRID_IQ2XXS : F == IQ2_XS ? NQ_GRID_IQ2XS : F == IQ2_S ? NQ_GRID_IQ2S
                                                                                     : NQ_GRID_IQ1S;
    }
    NQ_HD static const uint32_t *src4() { return F == IQ3_XXS ? NQ_GRID_IQ3XXS : NQ_GRID_IQ3S; }
};

// Kernel arguments for one launch (one chunk of whole blocks).
struct KArgs {
    const uint32_t *base;     // payload of this chunk, aligned down to 4 bytes
    const uint32_t *tr_base;  // "nvfp4" divisor words, aligned down to 4 bytes
    void *out;                // output element 0 of this chunk
    uint32_t mis;             // payload start - base (0..3)
    uint32_t last;            // last payload dword of this chunk, from base
    uint32_t tr_mis;          // first divisor's address - tr_base (0..3)
    uint32_t tr_last;         // last dword holding divisor bytes, from tr_base
    uint32_t nunits;          // units in this chunk
    uint32_t ndiv;            // "nvfp4": number of divisors (stacked sources)
    uint64_t u0;              // "nvfp4": tensor unit index of the chunk's first unit
    uint64_t gu;              // "nvfp4": units per divisor group (rows per source * K / 8)
};

// Output type codes: 0 binary32, 1 binary16, 2 bfloat16, 3 binary64 (the
// C ABI's), and 4: binary32 with non-temporal stores, the launcher's choice
// for short binary32 launches (NQ_F32_NT_UNITS).
NQ_HD constexpr bool ot_f32(int ot) { return ot == 0 || ot == 4; }
NQ_HD constexpr uint64_t ot_size(int ot) { return ot_f32(ot) ? 4u : ot == 3 ? 8u : 2u; }

// Non-temporal 16-byte stores (streamed past the caches) pay off when each
// store instruction of a wave covers whole cache lines: the 16-bit outputs,
// where 64 lanes write one contiguous 1 KiB run.  The 32/64-bit outputs write
// each line from two instructions and keep ordinary stores, except binary32
// launches below NQ_F32_NT_UNITS units (3 * 2^18, 6 M values; output type
// 4): over rotations whose payloads alone pass 1 GiB, non-temporal stores
// decoded [64, 4096] to [1024, 4096] tensors to binary32 13-24% faster and
// [2048, 4096] ones 11-15% slower, [8192, 4096] and larger ones 30-55%
// slower (q4_0, q4_k, q8_0, nvfp4, iq2_xxs on MI355X).  NQ_NT_STORE
// overrides: 0 never, 1 always, 2 (default) as described.
#ifndef NQ_NT_STORE
#define NQ_NT_STORE 2
#endif
#ifndef NQ_F32_NT_UNITS
#define NQ_F32_NT_UNITS (3u << 18)
#endif
template <int OT>
NQ_HD void vstore(void *p, u32x4 v) {
    constexpr bool nt = NQ_NT_STORE == 1 || (NQ_NT_STORE == 2 && (OT == 1 || OT == 2 || OT == 4));
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (nt) {
        __builtin_nontemporal_store(v, (u32x4 *)p);
        return;
    }
#endif
    *(u32x4 *)p = v;
}

// Output conversion and store of one unit (8 values) at element 8u.
// Conversion happens once, from the binary32 value, with round-to-nearest-
// even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 under the default round mode).
template <int OT, bool VEC>
NQ_HD void store8(void *out, uint32_t u, const float (&y)[8]) {
    const uint64_t e = 8ull * u;
    if constexpr (ot_f32(OT)) {
        float *o = (float *)out + e;
        if constexpr (VEC) {
            u32x4 a, b;
            a.x = __builtin_bit_cast(uint32_t, y[0]); a.y = __builtin_bit_cast(uint32_t, y[1]);
            a.z = __builtin_bit_cast(uint32_t, y[2]); a.w = __builtin_bit_cast(uint32_t, y[3]);
            b.x = __builtin_bit_cast(uint32_t, y[4]); b.y = __builtin_bit_cast(uint32_t, y[5]);
            b.z = __builtin_bit_cast(uint32_t, y[6]); b.w = __builtin_bit_cast(uint32_t, y[7]);
            vstore<OT>(o, a);
            vstore<OT>(o + 4, b);
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++) o[k] = y[k];
        }
    } else if constexpr (OT == 1 || OT == 2) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            f32x2 v;
            v.x = y[2 * k];
            v.y = y[2 * k + 1];
            if constexpr (OT == 2)
                w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
            else
                w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
        }
        uint16_t *o = (uint16_t *)out + e;
        if constexpr (VEC) {
            u32x4 a;
            a.x = w[0]; a.y = w[1]; a.z = w[2]; a.w = w[3];
            vstore<OT>(o, a);
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++) o[k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
        }
    } else {
        double *o = (double *)out + e;
        if constexpr (VEC) {
#pragma unroll
            for (int k = 0; k < 4; k++) {
                f64x2 v;
                v.x = (double)y[2 * k];
                v.y = (double)y[2 * k + 1];
                vstore<OT>(o + 2 * k, __builtin_bit_cast(u32x4, v));
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++) o[k] = (double)y[k];
        }
    }
}

// One value at element e, converted as store8 converts it.
template <int OT>
NQ_HD void store1(void *out, uint64_t e, float y) {
    if constexpr (ot_f32(OT)) {
        ((float *)out)[e] = y;
    } else if constexpr (OT == 1 || OT == 2) {
        f32x2 v;
        v.x = y;
        v.y = 0.0f;
        uint32_t w;
        if constexpr (OT == 2)
            w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        else
            w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
        ((uint16_t *)out)[e] = (uint16_t)w;
    } else {
        ((double *)out)[e] = (double)y;
    }
}

// Division of 31-bit numerators by d (1 <= d <= 2^30) as floor(n * m / 2^s):
// with l = ceil(log2 d), m = floor(2^(31+l) / d) + 1 and s = 31 + l this is
// exact for every 0 <= n < 2^31 (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, theorem 4.2 with N = 31);
// m < 2^32.  The host computes (m, s) once per launch.
NQ_HD inline void div_magic(uint64_t d, uint32_t *m, uint32_t *s) {
    uint32_t l = 0;
    while ((1ull << l) < d) l++;
    *m = (uint32_t)((1ull << (31 + l)) / d + 1);
    *s = 31 + l;
}

constexpr int WG = 256;  // threads per workgroup (4 wave64)

// ---------------------------------------------------------------------------
// LDS-staged decode.  A workgroup decodes one tile.  It copies a full tile's
// payload bytes into LDS with coalesced 16-byte loads, Stage::NK per thread
// (1 to 5, by format and tile size), all issued before the lookup tables are
// filled; after one barrier every thread decodes its units from LDS through
// LdsSrc with the same unit decoders the direct path uses.  Latency is hidden
// by the other workgroups resident on the compute unit, not by prefetching
// inside one.  Every global dword index is clamped to the last payload dword,
// so staging never leaves the payload.  The phases (stage_load, stage_store,
// decode_staged) are host-compilable so the emulator can run them in barrier
// order.
// ---------------------------------------------------------------------------

struct LdsSrc {
    const uint32_t *base;  // the staged tile: LDS dword 0 = payload dword a0
    uint32_t last;         // last staged dword holding this tile's bytes
    template <int N>
    NQ_HD void load(uint32_t i, uint32_t (&r)[N]) const {
#pragma unroll
        for (int k = 0; k < N; k++) r[k] = base[i + (uint32_t)k];
    }
    NQ_HD uint32_t dw(uint32_t i) const { return base[i]; }
    // the extra dword of a window: at most one past `last`, inside the slot's
    // padding, and unused there (no clamp needed)
    NQ_HD uint32_t dwx(uint32_t i) const {
#if !defined(__HIP_DEVICE_COMPILE__)
        if (i > last + 1) __builtin_trap();
#endif
        return base[i];
    }
};

// Cache policy of the staging loads, by launch size, measured on MI355X
// over rotations whose payloads alone pass 1 GiB (so every launch reads
// HBM):
//   - launches below NQ_STAGE_NT_UNITS units (6 * 2^20, 48 M values) load
//     non-temporally: 7-15% faster than ordinary loads at [1024, 4096] to
//     bf16, 0-6% at [4096, 4096] and [4096, 14336] (21 formats);
//   - longer launches take the format's choice (staging_nt): non-temporal
//     for the three 8-bit formats (q8_0, q8_1, q8_k), which read the most
//     payload bytes per value, and "nvfp4" (1-4% ahead at [14336, 4096]);
//     ordinary for the rest, which came within 2% either way at
//     [14336, 4096] but lost up to 5% non-temporally (q6_k, tq2_0) in the
//     long many-tensor launches of a weight set.
// The policy is a template argument of the kernels (two instantiations):
// under a run-time switch, two global loads that differ only in the
// non-temporal hint are merged by the compiler and lose it.
#ifndef NQ_STAGE_NT_UNITS
#define NQ_STAGE_NT_UNITS (6u << 20)
#endif
template <int F>
constexpr bool staging_nt() {
    return F == Q8_0 || F == Q8_1 || F == Q8_K || F == NVFP4_DIV;
}

template <int F>
NQ_HD bool stage_nt(uint64_t units) {
#if NQ_STAGE_NT >= 0
    (void)units;
    return NQ_STAGE_NT != 0;
#else
    return units < (uint64_t)NQ_STAGE_NT_UNITS || staging_nt<F>();
#endif
}

template <int F, int UPT>
struct Stage {
    static constexpr uint32_t UPB = block_values(F) / 8;
    static constexpr uint32_t PER = (uint32_t)(WG * UPT);      // units per tile
    static constexpr uint32_t BPT = PER / UPB;                  // blocks per tile
    static constexpr uint32_t TB = BPT * block_bytes(F);        // payload bytes per tile
    static constexpr uint32_t NDW = (TB + 3) / 4 + 1;           // dwords spanned, any start offset
    static constexpr uint32_t NCH = (NDW + 3) / 4;              // 16-byte chunks
    static constexpr uint32_t NK = (NCH + WG - 1) / WG;         // chunks per thread
    static constexpr uint32_t SLOT_DW = NCH * 4 + 4;            // LDS dwords per slot: chunks + padding
};

// Chunk c of tile t covers payload dwords a0 + 4c .. a0 + 4c + 3, where a0 is
// the tile's first dword; chunks 0..cmax hold the tile's bytes.  Threads
// whose chunk index passes cmax take chunk cmax again (same address within
// the wave, so no extra traffic, and the same value written to the same LDS
// dwords), which keeps the staging code free of branches.
template <int F, int UPT>
NQ_HD uint32_t stage_first(const KArgs &a, uint32_t t, uint32_t *cmax) {
    using ST = Stage<F, UPT>;
    const uint32_t p = a.mis + t * ST::TB;
    *cmax = (((p + ST::TB - 1) >> 2) - (p >> 2)) >> 2;
    return p >> 2;
}

// Tiles staged through LDS: the full tiles whose chunks all end at or before
// the last payload dword.  Only the last full tile can fail that (when no
// partial tile follows it); it then joins the tail.
template <int F, int UPT>
NQ_HD uint32_t staged_tiles(const KArgs &a) {
    using ST = Stage<F, UPT>;
    const uint32_t full = a.nunits / ST::PER;
    if (full == 0) return 0;
    uint32_t cmax;
    const uint32_t a0 = stage_first<F, UPT>(a, full - 1, &cmax);
    return a0 + 4u * cmax + 3u <= a.last ? full : full - 1;
}

// Global loads of tile t's chunks for this thread (into registers); t is a
// staged tile, so every chunk lies inside the payload.
template <int F, int UPT, bool NT, class Src>
NQ_HD void stage_load(const Src &src, const KArgs &a, uint32_t t, uint32_t tid, uint32_t (&r)[Stage<F, UPT>::NK][4]) {
    using ST = Stage<F, UPT>;
    uint32_t cmax;
    const uint32_t a0 = stage_first<F, UPT>(a, t, &cmax);
#pragma unroll
    for (uint32_t k = 0; k < ST::NK; k++) {
        const uint32_t c0 = k * WG + tid;
        src.template load4<NT>(a0 + 4u * (c0 < cmax ? c0 : cmax), r[k]);
    }
}

template <int F, int UPT>
NQ_HD void stage_store(uint32_t *slot, const KArgs &a, uint32_t t, uint32_t tid,
                       const uint32_t (&r)[Stage<F, UPT>::NK][4]) {
    using ST = Stage<F, UPT>;
    uint32_t cmax;
    stage_first<F, UPT>(a, t, &cmax);
#pragma unroll
    for (uint32_t k = 0; k < ST::NK; k++) {
        const uint32_t c0 = k * WG + tid;
        u32x4 v;
        v.x = r[k][0]; v.y = r[k][1]; v.z = r[k][2]; v.w = r[k][3];
        *(u32x4 *)(slot + 4u * (c0 < cmax ? c0 : cmax)) = v;
    }
}

// "nvfp4" units past the divisor group of the tile's first unit (u >=
// tab.nv_bound) are decoded a second time, dividing by their own group's
// divisor directly (the same correctly rounded quotient the table holds); the
// first pass skips their stores.  This pass is a rolled loop so that its
// divisions appear once in the code.
NQ_HD inline bool nv_table_unit(const Tab &tab, uint32_t u) { return u < tab.nv_bound; }

// Decode this thread's units of tile t from its staged copy in `buf`.  A
// block's units are consecutive and a tile row of 256 units holds whole
// blocks, so unit k*256 + tid of a tile lies in the tile's block
// k*(256/UPB) + tid/UPB, at unit tid % UPB of that block.
template <int F, int OT, int UPT, bool VEC, class T>
NQ_HD void decode_staged(const T &tab, const KArgs &a, uint32_t t, uint32_t tid, const uint32_t *buf) {
    using ST = Stage<F, UPT>;
    constexpr uint32_t UPB = ST::UPB;
    constexpr uint32_t S = block_bytes(F);
    static_assert(WG % UPB == 0, "a tile row holds whole blocks");
    const uint32_t p = a.mis + t * ST::TB;
    const uint32_t a0 = p >> 2;
    const LdsSrc src{buf, ((p + ST::TB - 1) >> 2) - a0};
    const uint32_t s = tid % UPB;
    const uint32_t bo0 = (p & 3u) + (tid / UPB) * S;
#pragma unroll
    for (int k = 0; k < UPT; k++) {
        const uint32_t u = t * ST::PER + (uint32_t)(k * WG) + tid;
        float y[8];
        decode_unit<F>(src, bo0 + (uint32_t)k * (WG / UPB) * S, s, tab, y);
        if (F != NVFP4_DIV || nv_table_unit(tab, u)) store8<OT, VEC>(a.out, u, y);
    }
    if constexpr (F == NVFP4_DIV) {
        if (!nv_table_unit(tab, t * ST::PER + (uint32_t)((UPT - 1) * WG) + tid)) {
#pragma unroll 1
            for (int k = 0; k < UPT; k++) {
                const uint32_t u = t * ST::PER + (uint32_t)(k * WG) + tid;
                if (nv_table_unit(tab, u)) continue;
                float y[8];
                unit_nvfp4_div<true>(src, bo0 + (uint32_t)k * (WG / UPB) * S, s, tab,
                                     tab.nvd[1u + (u - tab.nv_bound) / tab.nv_gu], y);
                store8<OT, VEC>(a.out, u, y);
            }
        }
    }
}

// A tile that is not staged (a partial last tile, or the last full tile when
// its chunks would pass the payload's end), decoded straight from global
// memory.
template <int F, int OT, int UPT, bool VEC, class Src, class T>
NQ_HD void decode_direct(const Src &src, const T &tab, const KArgs &a, uint32_t t, uint32_t tid) {
    using ST = Stage<F, UPT>;
#pragma unroll
    for (int k = 0; k < UPT; k++) {
        const uint32_t u = t * ST::PER + (uint32_t)(k * WG) + tid;
        if (u < a.nunits) {
            float y[8];
            decode_unit<F>(src, a.mis + (u / ST::UPB) * block_bytes(F), u % ST::UPB, tab, y);
            if (F != NVFP4_DIV || nv_table_unit(tab, u)) store8<OT, VEC>(a.out, u, y);
        }
    }
    if constexpr (F == NVFP4_DIV) {
#pragma unroll 1
        for (int k = 0; k < UPT; k++) {
            const uint32_t u = t * ST::PER + (uint32_t)(k * WG) + tid;
            if (u >= a.nunits || nv_table_unit(tab, u)) continue;
            float y[8];
            unit_nvfp4_div<true>(src, a.mis + (u / ST::UPB) * block_bytes(F), u % ST::UPB, tab,
                                 tab.nvd[1u + (u - tab.nv_bound) / tab.nv_gu], y);
            store8<OT, VEC>(a.out, u, y);
        }
    }
}

// "nvfp4" divisor g (little-endian binary32 word g of the divisor array).
template <class TrSrc>
NQ_HD float divisor_at(const TrSrc &tr, const KArgs &a, uint32_t g) {
    uint32_t w[1];
    window<1>(tr, a.tr_mis + 4u * g, w);
    return bits_f32(w[0]);
}

// "nvfp4": d_w's sign bit in bit 7 of every byte (the sign the table's
// magnitudes lose).
NQ_HD uint32_t nv_sign_bytes(float dw) { return (__builtin_bit_cast(uint32_t, dw) >> 31) ? 0x80808080u : 0u; }

// "nvfp4": the divisor group of tile t's first unit, and the chunk-relative
// unit where that group ends (capped at 2^32 - 1).
template <int UPT>
NQ_HD uint32_t nv_first_group(const KArgs &a, uint32_t t, uint32_t *bound) {
    if (a.ndiv == 1) {  // one divisor: skip the 64-bit division
        *bound = 0xFFFFFFFFu;
        return 0;
    }
    const uint64_t g0 = (a.u0 + (uint64_t)t * (uint32_t)(WG * UPT)) / a.gu;
    const uint64_t end = (g0 + 1) * a.gu - a.u0;
    *bound = end > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)end;
    return (uint32_t)g0;
}

// Table setup for the tile whose first divisor group is g0, strided over
// `nthreads` cooperating threads.
template <int F, class TrSrc>
NQ_HD void fill_tables(uint64_t *t8, uint32_t *t4, float *nvq, float *nvd, const TrSrc &tr, const KArgs &a,
                       uint32_t g0, uint32_t tid, uint32_t nthreads) {
    using TS = TabSpec<F>;
    if constexpr (TS::n8 > 0) {
        const uint64_t *g = TS::src8();
        for (uint32_t r = tid; r < (uint32_t)TS::n8; r += nthreads) t8[r] = g[r];
    }
    if constexpr (TS::n4 > 0) {
        const uint32_t *g = TS::src4();
        for (uint32_t r = tid; r < (uint32_t)TS::n4; r += nthreads) t4[r] = g[r];
    }
    if constexpr (TS::nf > 0) {
        const uint32_t nd = a.ndiv - g0 < (uint32_t)TS::nd ? a.ndiv - g0 : (uint32_t)TS::nd;
        for (uint32_t k = tid; k < nd; k += nthreads) nvd[k] = divisor_at(tr, a, g0 + k);
        const float dw = divisor_at(tr, a, g0);
        for (uint32_t k = tid; k < (uint32_t)TS::nf / 4u; k += nthreads) {
            uint32_t e[4], code[4];
            nvfp4_table_quad(k >> 1, k & 1u, dw, e, code);
#pragma unroll
            for (int i = 0; i < 4; i++) nvq[8u * (k >> 1) + code[i]] = bits_f32(e[i]);
        }
    }
}

// Tile t of the launch described by `a`: staged in LDS and decoded (or
// decoded from global memory when it is not staged).  The tile's loads are
// issued before the lookup tables are filled, so the two latencies overlap,
// and one barrier publishes both.  The LDS arrays are the kernel's.
template <int F, int OT, int UPT, bool VEC, bool NT>
__device__ __forceinline__ void decode_tile(const KArgs &a, uint32_t t, uint32_t tid, uint64_t *t8, uint32_t *t4,
                                            float *nvq, float *nvd, uint32_t *lds) {
    using TS = TabSpec<F>;
    using ST = Stage<F, UPT>;
    const DevSrc src{a.base, a.last};
    Tab tab{t8, t4, nvq, nvd, 0xFFFFFFFFu, 1u, 0u};
    uint32_t g0 = 0;
    const DevSrc tr{a.tr_base, a.tr_last};
    if constexpr (F == NVFP4_DIV) {
        g0 = nv_first_group<UPT>(a, t, &tab.nv_bound);
        tab.nv_gu = a.gu < 0x7FFFFFFFull ? (uint32_t)a.gu : 0x7FFFFFFFu;
        tab.nv_dsign = nv_sign_bytes(divisor_at(tr, a, g0));
    }
    if (t < staged_tiles<F, UPT>(a)) {
        uint32_t r[ST::NK][4];
        stage_load<F, UPT, NT>(src, a, t, tid, r);
        if constexpr (TS::n8 + TS::n4 + TS::nf > 0) fill_tables<F>(t8, t4, nvq, nvd, tr, a, g0, tid, WG);
        stage_store<F, UPT>(lds, a, t, tid, r);
        __syncthreads();
        decode_staged<F, OT, UPT, VEC>(tab, a, t, tid, lds);
    } else {
        if constexpr (TS::n8 + TS::n4 + TS::nf > 0) {
            fill_tables<F>(t8, t4, nvq, nvd, tr, a, g0, tid, WG);
            __syncthreads();
        }
        decode_direct<F, OT, UPT, VEC>(src, tab, a, t, tid);
    }
}

// The LDS of one decode workgroup: lookup tables and the staged tile.
#define NQ_DECODE_LDS(F, UPT)                                                   \
    __shared__ uint64_t t8[TabSpec<F>::n8 > 0 ? TabSpec<F>::n8 : 1];            \
    __shared__ uint32_t t4[TabSpec<F>::n4 > 0 ? TabSpec<F>::n4 : 1];            \
    __shared__ float nvq[TabSpec<F>::nf > 0 ? TabSpec<F>::nf : 1];              \
    __shared__ float nvd[TabSpec<F>::nd > 0 ? TabSpec<F>::nd : 1];              \
    __shared__ __attribute__((aligned(16))) uint32_t lds[Stage<F, UPT>::SLOT_DW]

// One workgroup per tile: workgroup t decodes tile t; the hardware keeps as
// many workgroups in flight as LDS and registers allow.  STACKED: an "nvfp4"
// launch with more than one divisor; otherwise the divisor count is the
// constant 1, and the code for units past the first divisor group compiles
// away (that code cost the one-divisor decode 10-15%).  NT: non-temporal
// staging loads (stage_nt).
template <int F, int OT, int UPT, bool VEC, bool STACKED, bool NT>
__global__ __launch_bounds__(WG) void k_decode(KArgs a) {
    NQ_DECODE_LDS(F, UPT);
    if constexpr (!STACKED) a.ndiv = 1;
    decode_tile<F, OT, UPT, VEC, NT>(a, blockIdx.x, threadIdx.x, t8, t4, nvq, nvd, lds);
}

// ---------------------------------------------------------------------------
// Several tensors of one format and output type in one launch
// (nq_dequantize_packed_many).  Each tensor (or launch chunk of one) keeps
// its own tiles, numbered on from the previous tensor's; a workgroup finds
// its tensor by a binary search over the first-tile numbers, which are
// uniform, so the search runs on scalar registers.  Decoding a unit does not
// depend on the tile it sits in, so every value is the one a single-tensor
// launch gives.
// ---------------------------------------------------------------------------
constexpr int MANY_MAX = 64;  // tensors (or chunks of tensors) per launch

struct MTensor {
    const uint32_t *base;     // payload, aligned down to 4 bytes
    const uint32_t *tr_base;  // "nvfp4": the divisor word, aligned down to 4 bytes
    void *out;                // output element 0
    uint32_t mis, last;       // as KArgs
    uint32_t tr_mis, tr_last; // as KArgs
    uint32_t nunits;          // units of this tensor (chunk)
    uint32_t tile0;           // its first tile, counted over the launch
};

struct MArgs {
    uint32_t n;  // entries used
    uint32_t ntiles;
    MTensor t[MANY_MAX];
};
static_assert(sizeof(MArgs) <= 4096, "kernel arguments stay within 4 KiB");

NQ_HD KArgs many_entry_args(const MTensor &e) {
    KArgs a;
    a.base = e.base;
    a.tr_base = e.tr_base;
    a.out = e.out;
    a.mis = e.mis;
    a.last = e.last;
    a.tr_mis = e.tr_mis;
    a.tr_last = e.tr_last;
    a.nunits = e.nunits;
    a.ndiv = 1;  // one divisor per "nvfp4" tensor
    a.u0 = 0;
    a.gu = e.nunits ? e.nunits : 1u;
    return a;
}

// Index of the entry holding tile b: the last entry whose first tile is at
// or before b (entries have at least one tile each).
NQ_HD uint32_t many_find(const MArgs &m, uint32_t b) {
    uint32_t lo = 0, hi = m.n;
    while (hi - lo > 1u) {
        const uint32_t mid = (lo + hi) >> 1;
        if (m.t[mid].tile0 <= b)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

template <int F, int OT, int UPT, bool VEC, bool NT>
__global__ __launch_bounds__(WG) void k_decode_many(MArgs m) {
    NQ_DECODE_LDS(F, UPT);
    const uint32_t b = blockIdx.x;
    const uint32_t j = many_find(m, b);
    const KArgs a = many_entry_args(m.t[j]);
    decode_tile<F, OT, UPT, VEC, NT>(a, b - m.t[j].tile0, threadIdx.x, t8, t4, nvq, nvd, lds);
}

// Host launch description for one call.
struct LaunchArgs {
    const uint8_t *payload;  // device
    uint64_t nbytes;
    uint64_t nblocks;
    void *out;               // device
    uint32_t resident;       // workgroups the device holds at once (the tile-size scale)
    uint32_t ndiv;           // "nvfp4": divisor words after the blocks (stacked sources)
    uint64_t gu;             // "nvfp4": units per divisor group
};


// Blocks per launch chunk: unit indices stay below 2^30 and payload byte
// offsets below 2^32.
template <int F>
constexpr uint64_t chunk_blocks() {
    constexpr uint64_t a = (1ull << 30) / (block_values(F) / 8), b = 0xFFFFFFF0ull / block_bytes(F);
    return a < b ? a : b;
}

// Kernel arguments and grid size of the chunk starting at block b0.
template <int F, int OT, int UPT>
NQ_HD KArgs chunk_args(const LaunchArgs &L, uint64_t b0, uint64_t nb, uint32_t *grid) {
    constexpr uint64_t S = block_bytes(F);
    constexpr uint64_t OSZ = ot_size(OT);
    const uint8_t *p = L.payload + b0 * S;
    const uint8_t *tr = L.payload + L.nbytes - (F == NVFP4_DIV ? 4ull * L.ndiv : 0);
    KArgs a;
    a.base = (const uint32_t *)((uintptr_t)p & ~(uintptr_t)3);
    a.mis = (uint32_t)((uintptr_t)p & 3);
    a.last = (uint32_t)((a.mis + nb * S - 1) >> 2);
    a.tr_base = (const uint32_t *)((uintptr_t)tr & ~(uintptr_t)3);
    a.tr_mis = (uint32_t)((uintptr_t)tr & 3);
    a.tr_last = F == NVFP4_DIV ? (uint32_t)((a.tr_mis + 4ull * L.ndiv - 1) >> 2) : 0u;
    a.ndiv = F == NVFP4_DIV ? L.ndiv : 0u;
    a.u0 = b0 * (block_values(F) / 8);
    a.gu = F == NVFP4_DIV ? L.gu : 1u;
    a.nunits = (uint32_t)(nb * (block_values(F) / 8));
    a.out = (uint8_t *)L.out + b0 * (uint64_t)block_values(F) * OSZ;
    const uint64_t per_wg = (uint64_t)WG * UPT;
    *grid = (uint32_t)((a.nunits + per_wg - 1) / per_wg);  // one workgroup per tile
    return a;
}

// Units per thread per tile for a launch of `nunits` units.  With R the
// workgroups the device holds at once (`resident`; 2048 on MI355X) and
// tiles(u) = ceil(nunits / (256 u)) the launch's workgroups at u units per
// thread, the choice counts rounds of R workgroups:
//   - q = nunits / R below 128: 1 (under half a round even then);
//   - tiles(L) >= 4R, L the format's long-launch size (upt_long): L.  Many
//     rounds of small tiles: the workgroups drift apart, so loads and stores
//     of several tiles are in flight on every compute unit throughout;
//   - else the smallest of 2 (4 for "nvfp4", upt_first), 4, 8 whose tiles
//     fit in one round, if one does: the whole launch starts at once, in as
//     many workgroups as fit;
//   - else L.
// One to three rounds run nearly in step: each round starts only as the one
// before drains, which left a launch of two rounds of 2-unit tiles 20% slower
// than one round of 4-unit tiles ([4096, 4096] tensors to bf16, formats q4_0,
// q4_k, q6_k, mxfp4, gguf:nvfp4, iq4_xs on MI355X; rows from 1024 to 14336 at
// 4096 columns were measured for 12 formats and tile sizes 2, 4 and 8, over
// rotations whose payloads alone pass 1 GiB).  L is the size that decoded a
// [14336, 4096] tensor to bf16 fastest: smaller tiles keep more independent
// loads and stores in flight; formats whose workgroups copy a codebook or
// fill a quotient table, and those with few payload bytes per value (q2_k,
// tq2_0), do better with larger tiles.
// Large codebooks (IQ2_S, IQ1_S, IQ1_M, which copy 8-16 KiB to LDS per
// workgroup) keep a rule by q alone: q < 128 -> 1, < 256 -> 2, < 512 -> 4,
// else 8.  The upt_wide formats take 16 from q = 3072 on, ahead of both
// rules.  Outputs that are not 16-byte aligned, and f64 outputs, always take
// 8.  NQ_UPT, when defined, fixes the tile size of every launch; NQ_UPT_LONG
// replaces every format's L.
template <int F>
constexpr bool big_codebook() {
    return TabSpec<F>::n8 >= 1024;
}

template <int F>
constexpr int upt_long() {
#ifdef NQ_UPT_LONG
    return NQ_UPT_LONG;
#else
    return (F == Q2_K || F == Q3_K || F == IQ2_XXS || F == IQ2_XS || F == IQ3_XXS || F == IQ1_S || F == IQ3_S ||
            F == IQ2_S || F == IQ1_M || F == TQ1_0 || F == TQ2_0) ? 8
         : (F == Q5_0 || F == Q1_0 || F == Q2_0 || F == NVFP4_DIV) ? 4
         : 2;
#endif
}

// Formats whose long launches take 16-unit tiles (q >= 3072: a [14336, 4096]
// tensor in 1792 workgroups, one round): the ones that copy the largest
// codebooks to LDS per workgroup (IQ1_M, IQ1_S 16 KiB, IQ2_S 8 KiB, IQ2_XS
// 4 KiB) and IQ3_S.  To bf16 at [14336, 4096] they ran 6-9% faster than with
// 8-unit tiles over cold rotations; IQ2_XXS, IQ3_XXS and the formats without
// codebooks ran 3-13% slower.
template <int F>
constexpr bool upt_wide() {
    return F == IQ1_M || F == IQ1_S || F == IQ2_S || F == IQ2_XS || F == IQ3_S;
}

// The smallest tile size of the one-round choice: 4 for "nvfp4", whose
// workgroups each fill a quotient table (two divisions per scale value) that
// 2-unit tiles would fill once per 512 units, 2 otherwise.
template <int F>
constexpr int upt_first() {
    return F == NVFP4_DIV ? 4 : 2;
}

template <int F>
NQ_HD int choose_upt(uint64_t nunits, uint32_t resident) {
#ifdef NQ_UPT
    (void)nunits;
    (void)resident;
    return NQ_UPT;
#else
    const uint64_t R = resident ? resident : 1u;
    const uint64_t q = nunits / R;
    if (q < 128) return 1;
    if (upt_wide<F>() && q >= 3072) return 16;
    if constexpr (big_codebook<F>()) {
        const int u = q < 256 ? 2 : q < 512 ? 4 : 8;
        return u < upt_long<F>() ? u : upt_long<F>();
    } else {
        constexpr int L = upt_long<F>();
        auto tiles = [&](uint64_t u) { return (nunits + WG * u - 1) / (WG * u); };
        if (tiles(L) >= 4 * R) return L;
        for (int u = upt_first<F>(); u <= 8; u *= 2)
            if (tiles(u) <= R) return u;
        return L;
    }
#endif
}

#ifdef NQ_UPT
constexpr int UPT_FIXED = NQ_UPT;
#else
constexpr int UPT_FIXED = 8;
#endif

template <int F, int OT, int UPT, bool VEC>
int launch_chunk(const LaunchArgs &L, uint64_t b0, uint64_t nb, hipStream_t stream) {
    uint32_t grid;
    const KArgs a = chunk_args<F, OT, UPT>(L, b0, nb, &grid);
    const bool nt = stage_nt<F>(L.nblocks * (block_values(F) / 8));  // by the whole tensor's units
    if (F == NVFP4_DIV && a.ndiv > 1) {
        if (nt)
            hipLaunchKernelGGL((k_decode<F, OT, UPT, VEC, F == NVFP4_DIV, true>), dim3(grid), dim3(WG), 0, stream, a);
        else
            hipLaunchKernelGGL((k_decode<F, OT, UPT, VEC, F == NVFP4_DIV, false>), dim3(grid), dim3(WG), 0, stream, a);
    } else {
        if (nt)
            hipLaunchKernelGGL((k_decode<F, OT, UPT, VEC, false, true>), dim3(grid), dim3(WG), 0, stream, a);
        else
            hipLaunchKernelGGL((k_decode<F, OT, UPT, VEC, false, false>), dim3(grid), dim3(WG), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : 9;  // NQ_ERR_HIP
}

template <int F, int OT>
int launch(const LaunchArgs &L, hipStream_t stream) {
    if constexpr (OT == 0 && NQ_NT_STORE == 2)
        if (L.nblocks * (block_values(F) / 8) < (uint64_t)NQ_F32_NT_UNITS) return launch<F, 4>(L, stream);
    constexpr uint64_t CB = chunk_blocks<F>();
    constexpr uint64_t OSZ = ot_size(OT);
    for (uint64_t b0 = 0; b0 < L.nblocks; b0 += CB) {
        const uint64_t nb = (L.nblocks - b0 < CB) ? L.nblocks - b0 : CB;
        const uintptr_t out = (uintptr_t)L.out + b0 * (uint64_t)block_values(F) * OSZ;
        int st;
        if ((out & 15) != 0) {
            st = launch_chunk<F, OT, UPT_FIXED, false>(L, b0, nb, stream);
        } else if constexpr (OT == 3) {
            st = launch_chunk<F, OT, UPT_FIXED, true>(L, b0, nb, stream);
        } else {
#ifdef NQ_UPT
            st = launch_chunk<F, OT, UPT_FIXED, true>(L, b0, nb, stream);
#else
            switch (choose_upt<F>(nb * (block_values(F) / 8), L.resident)) {
            case 1: st = launch_chunk<F, OT, 1, true>(L, b0, nb, stream); break;
            case 2: st = launch_chunk<F, OT, 2, true>(L, b0, nb, stream); break;
            case 4: st = launch_chunk<F, OT, 4, true>(L, b0, nb, stream); break;
            case 8: st = launch_chunk<F, OT, 8, true>(L, b0, nb, stream); break;
            case 16:
                if constexpr (upt_wide<F>())
                    st = launch_chunk<F, OT, 16, true>(L, b0, nb, stream);
                else
                    st = 9;  // unreachable: only upt_wide formats take 16
                break;
            default: st = 9; break;  // unreachable: choose_upt returns 1, 2, 4, 8 or 16
            }
#endif
        }
        if (st != 0) return st;
    }
    return 0;
}

// One tensor of a many-tensor call: its payload, block count and output.
struct ManyItem {
    const uint8_t *payload;  // device
    uint64_t nbytes;
    uint64_t nblocks;
    void *out;               // device, 16-byte aligned when VEC
};

// Entries of the launch chunk of item `it` that starts at block b0 (nb blocks).
template <int F, int OT>
NQ_HD MTensor many_entry(const ManyItem &it, uint64_t b0, uint64_t nb) {
    LaunchArgs L;
    L.payload = it.payload;
    L.nbytes = it.nbytes;
    L.nblocks = it.nblocks;
    L.out = it.out;
    L.resident = 0;
    L.ndiv = 1;
    L.gu = 1;
    uint32_t grid;
    const KArgs a = chunk_args<F, OT, 1>(L, b0, nb, &grid);
    MTensor e;
    e.base = a.base;
    e.tr_base = a.tr_base;
    e.out = a.out;
    e.mis = a.mis;
    e.last = a.last;
    e.tr_mis = a.tr_mis;
    e.tr_last = a.tr_last;
    e.nunits = a.nunits;
    e.tile0 = 0;
    return e;
}

// Tiles of each entry for UPT units per thread, numbered from 0; false if the
// launch would pass 2^31 - 1 workgroups.
template <int UPT>
NQ_HD bool many_number_tiles(MArgs &m) {
    uint64_t t = 0;
    for (uint32_t j = 0; j < m.n; j++) {
        m.t[j].tile0 = (uint32_t)t;
        t += (m.t[j].nunits + (uint64_t)WG * UPT - 1) / ((uint64_t)WG * UPT);
        if (t > 0x7FFFFFFFull) return false;
    }
    m.ntiles = (uint32_t)t;
    return true;
}

template <int F, int OT, int UPT, bool VEC>
int launch_many_chunk(MArgs &m, bool nt, hipStream_t stream) {
    if (!many_number_tiles<UPT>(m)) return 9;  // NQ_ERR_HIP: cannot be launched as one grid
    if (nt)
        hipLaunchKernelGGL((k_decode_many<F, OT, UPT, VEC, true>), dim3(m.ntiles), dim3(WG), 0, stream, m);
    else
        hipLaunchKernelGGL((k_decode_many<F, OT, UPT, VEC, false>), dim3(m.ntiles), dim3(WG), 0, stream, m);
    return hipGetLastError() == hipSuccess ? 0 : 9;
}

// Launches of `n` non-empty tensors of format F to output type OT: entries
// are packed MANY_MAX to a launch (a tensor larger than one launch chunk
// takes several entries), and go(m, upt, nt) receives each launch's
// arguments with its units per thread and staging cache policy.  Both follow
// the units of each launch as for one tensor (choose_upt, stage_nt), the
// tile size limited to 2, 4 and 8 units per thread (1 becomes 2, 16 becomes 8).  VEC: every output
// is 16-byte aligned (otherwise, and for f64 outputs, always 8).  CB: blocks
// per launch chunk (chunk_blocks<F>(); smaller in the emulator).  Host code
// shared by the launcher and the emulator.
template <int F, int OT, bool VEC, class Go>
int many_plan(const ManyItem *items, int n, uint32_t resident, uint64_t CB, Go &&go) {
    MArgs m;
    m.n = 0;
    m.ntiles = 0;
    uint64_t units = 0;
    auto flush = [&]() -> int {
        if (m.n == 0) return 0;
        const int c = choose_upt<F>(units, resident);
        const int upt = (VEC && OT != 3) ? (c <= 2 ? 2 : c == 4 ? 4 : 8) : 8;
        const int st = go(m, upt, stage_nt<F>(units));
        m.n = 0;
        units = 0;
        return st;
    };
    for (int i = 0; i < n; i++) {
        for (uint64_t b0 = 0; b0 < items[i].nblocks; b0 += CB) {
            const uint64_t nb = items[i].nblocks - b0 < CB ? items[i].nblocks - b0 : CB;
            if (m.n == (uint32_t)MANY_MAX) {
                const int st = flush();
                if (st != 0) return st;
            }
            m.t[m.n++] = many_entry<F, OT>(items[i], b0, nb);
            units += nb * (block_values(F) / 8);
        }
    }
    return flush();
}

template <int F, int OT, bool VEC>
int launch_many(const ManyItem *items, int n, uint32_t resident, hipStream_t stream) {
    return many_plan<F, OT, VEC>(items, n, resident, chunk_blocks<F>(), [&](MArgs &m, int upt, bool nt) -> int {
        if constexpr (VEC && OT != 3) {
            if (upt == 2) return launch_many_chunk<F, OT, 2, VEC>(m, nt, stream);
            if (upt == 4) return launch_many_chunk<F, OT, 4, VEC>(m, nt, stream);
        }
        return launch_many_chunk<F, OT, 8, VEC>(m, nt, stream);
    });
}

template <int F>
int launch_many_any(int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t stream) {
    switch (ot) {
    case 0: return vec ? launch_many<F, 0, true>(items, n, resident, stream) : launch_many<F, 0, false>(items, n, resident, stream);
    case 1: return vec ? launch_many<F, 1, true>(items, n, resident, stream) : launch_many<F, 1, false>(items, n, resident, stream);
    case 2: return vec ? launch_many<F, 2, true>(items, n, resident, stream) : launch_many<F, 2, false>(items, n, resident, stream);
    default: return vec ? launch_many<F, 3, true>(items, n, resident, stream) : launch_many<F, 3, false>(items, n, resident, stream);
    }
}

template <int F>
int launch_any(int ot, const LaunchArgs &L, hipStream_t stream) {
    switch (ot) {
    case 0: return launch<F, 0>(L, stream);
    case 1: return launch<F, 1>(L, stream);
    case 2: return launch<F, 2>(L, stream);
    default: return launch<F, 3>(L, stream);
    }
}

}  // namespace nq
