// nq_emu.hip -- host emulator of the decode kernels (test infrastructure).
//
// Runs the kernels' own per-thread code (the staging, decode and store
// phases of nq_kernel.h, and the row-scaled FP8 thread of nq_fp8row.h) for
// every workgroup and thread of every launch chunk, sequentially on the CPU,
// with the launchers' own chunk and grid arithmetic.  The payload sources
// check that every dword read overlaps the payload bytes of its chunk; the
// caller checks the output guards.  Built host-only.
//
// Built in parts so the instantiations compile in parallel: a part compiled
// with -DNQ_EMU_PART=p -DNQ_EMU_PARTS=P instantiates the block formats whose
// id is p mod P and registers them in the dispatch table; the build without
// NQ_EMU_PART holds the table and the exported entry points.
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <vector>

#include "../../block_quantized_weight_nq_amd/csrc/nq_fp8row.h"
#include "../../block_quantized_weight_nq_amd/csrc/nq_gemm.h"
#include "../../block_quantized_weight_nq_amd/csrc/nq_gqenc.h"
#include "../../block_quantized_weight_nq_amd/csrc/nq_kernel.h"

namespace {

struct Check {
    uintptr_t lo, hi;  // valid payload byte range [lo, hi)
    long errors;
    char msg[256];
};

struct HostSrc {
    const uint32_t *base;
    uint32_t last;
    Check *chk;
    template <int N>
    void load(uint32_t i, uint32_t (&r)[N]) const {
        for (int k = 0; k < N; k++) r[k] = dw(i + (uint32_t)k);
    }
    void load_stream4(uint32_t i, uint32_t (&r)[4]) const { load<4>(i, r); }
    template <bool NT>
    void load4(uint32_t i, uint32_t (&r)[4]) const { load<4>(i, r); }
    uint32_t dwx(uint32_t i) const { return dw(i < last ? i : last); }
    uint32_t dw(uint32_t i) const {
        const uintptr_t a = (uintptr_t)(base + i);
        if (i > last || a + 4 <= chk->lo || a >= chk->hi) {
            if (chk->errors++ == 0)
                snprintf(chk->msg, sizeof chk->msg, "dword %u (last %u) at %#lx outside payload [%#lx, %#lx)",
                         i, last, (unsigned long)a, (unsigned long)chk->lo, (unsigned long)chk->hi);
        }
        return base[i];
    }
};

// The kernel's work on one tile, run thread by thread: the prologue (the
// divisor group of the tile's first unit and the tables; stale divisor slots
// poisoned), then for a staged tile every thread's staging into the LDS slot
// (with guard words past it) and every thread's decode (the barrier between),
// for other tiles every thread's decode from the payload.
template <int F, int OT, int UPT>
struct EmuTiles {
    using TS = nq::TabSpec<F>;
    using ST = nq::Stage<F, UPT>;
    static constexpr uint32_t GUARD = 64, GUARD_WORD = 0x5A5A5A5Au;
    std::vector<uint64_t> t8 = std::vector<uint64_t>(TS::n8 > 0 ? TS::n8 : 1);
    std::vector<uint32_t> t4 = std::vector<uint32_t>(TS::n4 > 0 ? TS::n4 : 1);
    std::vector<float> nvq = std::vector<float>(TS::nf > 0 ? TS::nf : 1);
    std::vector<float> nvd = std::vector<float>(TS::nd > 0 ? TS::nd : 1);
    std::vector<uint32_t> slot = std::vector<uint32_t>(ST::SLOT_DW + GUARD);
    long lds_errors = 0;

    void tile(const nq::KArgs &a, uint32_t t, Check &chk, Check &chk_tr) {
        using namespace nq;
        const HostSrc tr{a.tr_base, a.tr_last, &chk_tr};
        const HostSrc src{a.base, a.last, &chk};
        const bool vec = ((uintptr_t)a.out & 15) == 0;
        uint32_t g0 = 0;
        Tab tab{t8.data(), t4.data(), nvq.data(), nvd.data(), 0xFFFFFFFFu, 1u, 0u};
        if constexpr (F == NVFP4_DIV) {
            g0 = nv_first_group<UPT>(a, t, &tab.nv_bound);
            tab.nv_gu = a.gu < 0x7FFFFFFFull ? (uint32_t)a.gu : 0x7FFFFFFFu;
            tab.nv_dsign = nv_sign_bytes(divisor_at(tr, a, g0));
            std::fill(nvd.begin(), nvd.end(), bits_f32(0x7FA5A5A5u));
            std::fill(nvq.begin(), nvq.end(), bits_f32(0x7FA5A5A5u));  // a table word the fill misses is NaN
        }
        if (TS::n8 + TS::n4 + TS::nf > 0)
            for (uint32_t tid = 0; tid < (uint32_t)WG; tid++)
                fill_tables<F>(t8.data(), t4.data(), nvq.data(), nvd.data(), tr, a, g0, tid, WG);
        if (t < staged_tiles<F, UPT>(a)) {
            std::fill(slot.begin(), slot.begin() + ST::SLOT_DW, 0xA5A5A5A5u);  // stale words poison the result
            std::fill(slot.begin() + ST::SLOT_DW, slot.end(), GUARD_WORD);
            for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) {
                uint32_t r[ST::NK][4];
                stage_load<F, UPT, false>(src, a, t, tid, r);  // the policy changes no value
                stage_store<F, UPT>(slot.data(), a, t, tid, r);
            }
            for (uint32_t i = ST::SLOT_DW; i < ST::SLOT_DW + GUARD; i++)
                if (slot[i] != GUARD_WORD && lds_errors++ == 0)
                    snprintf(chk.msg, sizeof chk.msg, "staging wrote past the LDS slot (tile %u)", t);
            for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) {
                if (vec)
                    decode_staged<F, OT, UPT, true>(tab, a, t, tid, slot.data());
                else
                    decode_staged<F, OT, UPT, false>(tab, a, t, tid, slot.data());
            }
        } else {
            for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) {
                if (vec)
                    decode_direct<F, OT, UPT, true>(src, tab, a, t, tid);
                else
                    decode_direct<F, OT, UPT, false>(src, tab, a, t, tid);
            }
        }
    }
};

long report(Check &chk, Check &chk_tr, long lds_errors, char *err, int errlen) {
    long errors = 0;
    chk.errors += lds_errors;
    for (Check *c : {&chk, &chk_tr})
        if (c->errors) {
            if (errors == 0) snprintf(err, errlen, "%s", c->msg);
            errors += c->errors;
        }
    return errors;
}

// One launch chunk with UPT units per thread, as the kernel runs it: one
// workgroup per tile.
template <int F, int OT, int UPT>
long run_chunk(const nq::LaunchArgs &L, uint64_t b0, uint64_t nb, const uint8_t *payload, uint64_t nbytes,
               char *err, int errlen) {
    using namespace nq;
    constexpr uint64_t S = block_bytes(F);
    using ST = Stage<F, UPT>;
    uint32_t grid;
    const KArgs a = chunk_args<F, OT, UPT>(L, b0, nb, &grid);
    Check chk{(uintptr_t)(payload + b0 * S), (uintptr_t)(payload + (b0 + nb) * S), 0, {0}};
    Check chk_tr{(uintptr_t)(payload + nbytes - 4ull * L.ndiv), (uintptr_t)(payload + nbytes), 0, {0}};
    if (grid != (a.nunits + ST::PER - 1) / ST::PER) {
        snprintf(err, errlen, "grid %u is not one workgroup per tile", grid);
        return 1;
    }
    EmuTiles<F, OT, UPT> emu;
    for (uint32_t t = 0; t < grid; t++) emu.tile(a, t, chk, chk_tr);
    return report(chk, chk_tr, emu.lds_errors, err, errlen);
}

// A many-tensor launch as the kernel runs it: every workgroup b of the grid
// finds its entry with the kernel's search and decodes that entry's tile
// b - tile0, its reads checked against that entry's payload bytes (and
// divisor).  Also checks that the search lands on the entry whose tiles hold
// b, and that the grid is the sum of the entries' tiles.
template <int F, int OT, int UPT>
long run_many_launch(const nq::MArgs &m, char *err, int errlen) {
    using namespace nq;
    constexpr uint64_t S = block_bytes(F), UPB = block_values(F) / 8;
    using ST = Stage<F, UPT>;
    EmuTiles<F, OT, UPT> emu;
    long errors = 0;
    uint64_t tiles = 0;
    for (uint32_t j = 0; j < m.n; j++) tiles += (m.t[j].nunits + ST::PER - 1) / ST::PER;
    if (tiles != m.ntiles || m.n == 0 || m.t[0].tile0 != 0) {
        snprintf(err, errlen, "grid %u for %llu tiles of %u entries", m.ntiles, (unsigned long long)tiles, m.n);
        return 1;
    }
    for (uint32_t b = 0; b < m.ntiles; b++) {
        const uint32_t j = many_find(m, b);
        const uint32_t end = j + 1 < m.n ? m.t[j + 1].tile0 : m.ntiles;
        if (b < m.t[j].tile0 || b >= end) {
            snprintf(err, errlen, "tile %u found entry %u with tiles [%u, %u)", b, j, m.t[j].tile0, end);
            return 1;
        }
        const KArgs a = many_entry_args(m.t[j]);
        const uintptr_t lo = (uintptr_t)a.base + a.mis, trlo = (uintptr_t)a.tr_base + a.tr_mis;
        Check chk{lo, lo + (uint64_t)a.nunits / UPB * S, 0, {0}};
        Check chk_tr{trlo, trlo + (F == NVFP4_DIV ? 4u : 0u), 0, {0}};
        const long lds_before = emu.lds_errors;
        emu.tile(a, b - m.t[j].tile0, chk, chk_tr);
        const long e = report(chk, chk_tr, emu.lds_errors - lds_before, err, errlen);
        if (e && errors == 0) errors = e;
        else errors += e;
    }
    return errors;
}

// The many-tensor launcher's packing (many_plan) and every launch it makes.
// *launches_out: launches made; *upt_mask: bit u set when a launch took u
// units per thread.
template <int F, int OT>
long run_many(const nq::ManyItem *items, int n, uint32_t resident, uint64_t chunk, int *launches_out, int *upt_mask,
              char *err, int errlen) {
    using namespace nq;
    long errors = 0;
    *launches_out = 0;
    *upt_mask = 0;
    auto go = [&](MArgs &m, int upt, bool) -> int {
        (*launches_out)++;
        *upt_mask |= 1 << upt;
        long e;
        if (upt == 2) {
            if (!many_number_tiles<2>(m)) return 9;
            e = run_many_launch<F, OT, 2>(m, err, errlen);
        } else if (upt == 4) {
            if (!many_number_tiles<4>(m)) return 9;
            e = run_many_launch<F, OT, 4>(m, err, errlen);
        } else {
            if (!many_number_tiles<8>(m)) return 9;
            e = run_many_launch<F, OT, 8>(m, err, errlen);
        }
        errors += e;
        return 0;
    };
    const bool vec = n > 0 && ((uintptr_t)items[0].out & 15) == 0;
    const uint64_t cb = chunk ? chunk : chunk_blocks<F>();
    const int st = vec ? many_plan<F, OT, true>(items, n, resident, cb, go)
                       : many_plan<F, OT, false>(items, n, resident, cb, go);
    if (st != 0) {
        snprintf(err, errlen, "launch plan failed with status %d", st);
        return 1;
    }
    return errors;
}

template <int F>
long run_many_ot(int ot, const nq::ManyItem *items, int n, uint32_t resident, uint64_t chunk, int *launches,
                 int *upt_mask, char *err, int errlen) {
    switch (ot) {
    case 0: return run_many<F, 0>(items, n, resident, chunk, launches, upt_mask, err, errlen);
    case 1: return run_many<F, 1>(items, n, resident, chunk, launches, upt_mask, err, errlen);
    case 2: return run_many<F, 2>(items, n, resident, chunk, launches, upt_mask, err, errlen);
    default: return run_many<F, 3>(items, n, resident, chunk, launches, upt_mask, err, errlen);
    }
}

// The launcher's chunk loop and per-chunk choice of units per thread
// (force_upt > 0 overrides the choice for aligned outputs).
template <int F, int OT>
long run(const uint8_t *payload, uint64_t nbytes, uint64_t nblocks, void *out, uint32_t max_wgs,
         uint64_t chunk, int force_upt, uint32_t ndiv, char *err, int errlen) {
    using namespace nq;
    const uint64_t units = nblocks * (block_values(F) / 8);
    LaunchArgs L{payload, nbytes, nblocks, out, max_wgs, ndiv, units / ndiv ? units / ndiv : 1};
    const uint64_t CB = chunk ? chunk : chunk_blocks<F>();
    constexpr uint64_t OSZ = OT == 0 ? 4 : OT == 3 ? 8 : 2;
    long errors = 0;
    for (uint64_t b0 = 0; b0 < nblocks; b0 += CB) {
        const uint64_t nb = (nblocks - b0 < CB) ? nblocks - b0 : CB;
        const uintptr_t o = (uintptr_t)out + b0 * (uint64_t)block_values(F) * OSZ;
        int upt = UPT_FIXED;  // misaligned and f64 outputs
        if ((o & 15) == 0 && OT != 3)
            upt = force_upt > 0 ? force_upt : choose_upt<F>(nb * (block_values(F) / 8), max_wgs);
        long e;
        switch (upt) {
        case 1: e = run_chunk<F, OT, 1>(L, b0, nb, payload, nbytes, err, errlen); break;
        case 2: e = run_chunk<F, OT, 2>(L, b0, nb, payload, nbytes, err, errlen); break;
        case 4: e = run_chunk<F, OT, 4>(L, b0, nb, payload, nbytes, err, errlen); break;
        case 8: e = run_chunk<F, OT, 8>(L, b0, nb, payload, nbytes, err, errlen); break;
        case 16: e = run_chunk<F, OT, 16>(L, b0, nb, payload, nbytes, err, errlen); break;
        default: snprintf(err, errlen, "no tile size %d", upt); return 1;
        }
        errors += e;
    }
    return errors;
}

template <int F>
long run_ot(int ot, const uint8_t *p, uint64_t nbytes, uint64_t nblocks, void *out, uint32_t mw, uint64_t ch,
            int fu, uint32_t nd, char *err, int errlen) {
    switch (ot) {
    case 0: return run<F, 0>(p, nbytes, nblocks, out, mw, ch, fu, nd, err, errlen);
    case 1: return run<F, 1>(p, nbytes, nblocks, out, mw, ch, fu, nd, err, errlen);
    case 2: return run<F, 2>(p, nbytes, nblocks, out, mw, ch, fu, nd, err, errlen);
    default: return run<F, 3>(p, nbytes, nblocks, out, mw, ch, fu, nd, err, errlen);
    }
}

template <int F>
long tile_blocks(int upt) {
    using namespace nq;
    switch (upt) {
    case 1: return (long)Stage<F, 1>::BPT;
    case 2: return (long)Stage<F, 2>::BPT;
    case 4: return (long)Stage<F, 4>::BPT;
    case 8: return (long)Stage<F, 8>::BPT;
    case 16: return (long)Stage<F, 16>::BPT;
    default: return -1;
    }
}

// The kernel's DPP wave sum, step by step: each step adds to every lane of
// the enabled rows the value its DPP source lane held before the step
// (disabled rows add +0); returns lane 63.
float dpp_sum63(float (&v)[64]) {
    auto step = [&](auto src_of, unsigned rows) {
        float t[64];
        for (int l = 0; l < 64; l++) t[l] = (rows >> (l >> 4)) & 1u ? v[src_of(l)] : 0.0f;
        for (int l = 0; l < 64; l++) v[l] = v[l] + t[l];
    };
    step([](int l) { return (l & ~3) | (l & 3) ^ 1; }, 0xFu);        // quad_perm [1,0,3,2]
    step([](int l) { return (l & ~3) | (l & 3) ^ 2; }, 0xFu);        // quad_perm [2,3,0,1]
    step([](int l) { return (l & ~7) | (7 - (l & 7)); }, 0xFu);      // row_half_mirror
    step([](int l) { return (l & ~15) | (15 - (l & 15)); }, 0xFu);   // row_mirror
    step([](int l) { return (l & ~15) - 1; }, 0xAu);                  // row_bcast:15 (rows 1, 3)
    step([](int l) { return 31; }, 0xCu);                             // row_bcast:31 (rows 2, 3)
    return v[63];
}

// Products with q8_1 activations: the launcher's row launches (max_rows > 0
// overrides the launcher's limit) and, per launch, a grid of `resident`
// workgroups (capped as the launcher caps it): the workgroup's activation
// staging and tables, then every wave's chunk sequence as the kernel walks
// it: the lanes' loads (through a bounds-checked source) and stores into a
// poisoned LDS region, whose bytes are then compared with the payload, the
// lanes' items, and at each row's end the wave's butterfly sum in the
// kernel's order.
template <int F, int MT, bool ALDS, int RW>
long run_gemv_lds(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y,
                  uint32_t resident, uint64_t max_rows, char *err, int errlen) {
    using namespace nq;
    const GvLaunch L{w, N, K, M, xq, y, 0u};
    const uint64_t lim = max_rows ? max_rows : gv_max_rows<F>(L);
    const uint64_t row_bytes = K / (uint64_t)block_values(F) * (uint64_t)block_bytes(F);
    std::vector<uint64_t> t8(TabSpec<F>::n8 > 0 ? TabSpec<F>::n8 : 1);
    std::vector<uint32_t> t4(TabSpec<F>::n4 > 0 ? TabSpec<F>::n4 : 1);
    for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) gv_fill_tables<F>(t8.data(), t4.data(), tid);
    const Tab tab{t8.data(), t4.data(), nullptr, nullptr, 0xFFFFFFFFu, 1u};
    long errors = 0;
    for (uint64_t r0 = 0; r0 < N;) {
        const uint64_t rows = N - r0 < lim ? N - r0 : lim;
        const GvArgs a = gv_args<F>(L, r0, rows);
        if (a.rw != (uint32_t)RW) {
            snprintf(err, errlen, "rows per chunk %u, kernel built for %d", a.rw, RW);
            return 1;
        }
        const uint32_t lds_bytes = gv_lds_bytes(a, ALDS);
        if (lds_bytes > 65536u) {
            snprintf(err, errlen, "LDS request %u bytes", lds_bytes);
            return 1;
        }
        const uint32_t grid = gv_grid(a, resident);
        Check chk{(uintptr_t)(w + r0 * row_bytes), (uintptr_t)(w + (r0 + rows) * row_bytes), 0, {0}};
        const HostSrc src{a.wbase, a.wlast, &chk};
        std::vector<uint32_t> act_lds(ALDS ? gv_act_dw(a) : 1u, 0xA5A5A5A5u);
        if (ALDS)
            for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) gv_stage_act(a, act_lds.data(), tid, WG);
        const GvAct<ALDS> act{a.xq, act_lds.data(), a.K, a.kb, a.xrow, a.M};
        std::vector<uint32_t> lds(gv_wave_dw<RW>());
        constexpr int NL = gv_nl<RW>();
        const uint32_t step = grid * GV_WAVES;
        for (uint32_t b = 0; b < grid; b++)
            for (uint32_t wave = 0; wave < GV_WAVES; wave++) {
                uint32_t r = (b * GV_WAVES + wave) * a.rw, c0 = 0;
                if (r >= a.rows) continue;
                static float acc[64][RW][MT];
                for (uint32_t lane = 0; lane < 64u; lane++)
                    for (int rr = 0; rr < RW; rr++)
                        for (int m = 0; m < MT; m++) acc[lane][rr][m] = 0.0f;
                GvChunk cur = gv_chunk(a, r, c0);
                for (;;) {
                    if (cur.g1 - cur.g0 + 1u > 64u * NL) {
                        snprintf(err, errlen, "chunk of %u groups past the wave's loads", cur.g1 - cur.g0 + 1u);
                        return 1;
                    }
                    std::fill(lds.begin(), lds.end(), 0xA5A5A5A5u);
                    for (uint32_t lane = 0; lane < 64u; lane++) {
                        uint32_t v[NL][4];
                        gv_issue<NL>(src, a.wlast, cur, lane, v);
                        gv_put<NL>(cur, a.wlast, lane, v, lds.data());
                    }
                    for (uint32_t rr = 0; rr < cur.rw; rr++) {
                        const uint8_t *cb = (const uint8_t *)lds.data() + cur.o0 + rr * a.row_bytes;
                        const uint8_t *pb = (const uint8_t *)a.wbase + a.wmis + (uint64_t)(cur.r + rr) * a.row_bytes +
                                            (uint64_t)cur.c0 * block_bytes(F);
                        if (memcmp(cb, pb, (size_t)cur.nb * block_bytes(F)) != 0 && chk.errors++ == 0)
                            snprintf(chk.msg, sizeof chk.msg, "staged chunk of row %u differs from the payload",
                                     cur.r + rr);
                    }
                    const LdsSrc s{lds.data(), 4u * (cur.g1 - cur.g0) + 3u};
                    for (uint32_t lane = 0; lane < 64u; lane++)
                        gv_chunk_items<F, MT, RW>(s, cur, lane, a.M, a.row_bytes, act, tab, acc[lane]);
                    if (cur.c0 + cur.nb >= a.nbr) {
                        for (uint32_t rr = 0; rr < cur.rw; rr++)
                            for (int m = 0; m < MT; m++) {
                                float v[64];
                                for (int l = 0; l < 64; l++) v[l] = acc[l][rr][m];
                                if (m < (int)a.M) a.y[(uint64_t)m * a.ldy + cur.r + rr] = dpp_sum63(v);
                            }
                        for (uint32_t lane = 0; lane < 64u; lane++)
                            for (int rr = 0; rr < RW; rr++)
                                for (int m = 0; m < MT; m++) acc[lane][rr][m] = 0.0f;
                    }
                    gv_advance(a, step, &r, &c0);
                    if (r >= a.rows) break;
                    cur = gv_chunk(a, r, c0);
                }
            }
        if (chk.errors) {
            if (errors == 0) snprintf(err, errlen, "%s", chk.msg);
            errors += chk.errors;
        }
        r0 += rows;
    }
    return errors;
}

// The emulator's device model of a compute unit: at most `limit`
// workgroups, 160 KiB of LDS and 32 waves (eight per SIMD).
int gv1_emu_per_cu(uint32_t limit, uint32_t nw, uint32_t lds) {
    const uint32_t by_lds = nq::GV1_LDS_MAX / lds, by_waves = 32u / nw;
    uint32_t n = limit < by_lds ? limit : by_lds;
    return (int)(n < by_waves ? n : by_waves);
}

// Phase-1 staging of a single-round workgroup as gv1_stage spreads it:
// load i of wave w moves group 64 * (i * nw + w) + lane of ng; every group
// must be moved exactly once.  Returns false (with a message) otherwise.
bool gv1_stage_cover(uint32_t ng, uint32_t nw, std::vector<uint32_t> &hits) {
    hits.assign(ng, 0u);
    for (uint32_t w = 0; w < nw; w++)
        for (uint32_t b = 64u * w; b < ng; b += 64u * nw)
            for (uint32_t lane = 0; lane < 64u; lane++)
                if (b + lane < ng) hits[b + lane]++;
    for (uint32_t q = 0; q < ng; q++)
        if (hits[q] != 1u) return false;
    return true;
}

// The single-round product kernel (k_gemv1) for a plan the launcher made.
// Per workgroup of p.nw waves: phase 1, the activation blocks (one
// activation row; several are read from global memory) and codebook tables
// moved into LDS as gv1_stage spreads them (coverage checked) and the
// activation blocks' code sums formed by the threads, then
// every wave's one chunk (p.rw whole rows, or part h of a row split in KS
// parts of p.cb blocks), staged as the kernel stages it (the 16-byte loads
// to LDS of groups g0 .. g1, each at a 16-byte aligned address and inside
// the payload, and the last group's shifted load) into a poisoned region
// whose size the plan gives; the staged bytes are compared with the
// payload; the count of chunk loads the wave waits on is checked against
// the loads that have an active lane; then the lanes' items (activation
// from the LDS copy) and each chunk row's butterfly sum, and for split rows
// the parts' sums added in part order by part 0's wave.
template <int F, int MT, int RW, int KS>
long run_gemv1(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y,
               const nq::Gv1Plan &p, char *err, int errlen) {
    using namespace nq;
    static_assert(KS == 1 || RW == 1, "a split row is a single-row chunk");
    const GvLaunch L{w, N, K, M, xq, y, 0u};
    std::vector<uint64_t> t8(TabSpec<F>::n8 > 0 ? TabSpec<F>::n8 : 1);
    std::vector<uint32_t> t4(TabSpec<F>::n4 > 0 ? TabSpec<F>::n4 : 1);
    std::vector<uint32_t> hits;
    if ((TabSpec<F>::n8 > 0 && !gv1_stage_cover(2u * (uint32_t)TabSpec<F>::n8, p.nw, hits)) ||
        (TabSpec<F>::n4 > 0 && !gv1_stage_cover((uint32_t)TabSpec<F>::n4, p.nw, hits))) {
        snprintf(err, errlen, "table staging does not cover every dword once");
        return 1;
    }
    if constexpr (TabSpec<F>::n8 > 0)
        memcpy(t8.data(), TabSpec<F>::src8(), sizeof(uint64_t) * (size_t)TabSpec<F>::n8);
    if constexpr (TabSpec<F>::n4 > 0)
        memcpy(t4.data(), TabSpec<F>::src4(), sizeof(uint32_t) * (size_t)TabSpec<F>::n4);
    const Tab tab{t8.data(), t4.data(), nullptr, nullptr, 0xFFFFFFFFu, 1u};
    GvArgs a = gv_args<F>(L, 0, N);
    a.rw = (uint32_t)RW;
    a.cb = p.cb;
    if (a.wmis != 0u || ((uintptr_t)a.wbase & 15u) != 0u || ((uintptr_t)xq & 15u) != 0u) {
        snprintf(err, errlen, "single-round launch on weight or activation bytes not 16-byte aligned");
        return 1;
    }
    const uint64_t chunks = KS == 1 ? (N + RW - 1) / RW : N * KS;
    if (p.lds != 4u * (gv1_act_region(p.act_dw) + p.nw * p.region_dw) || p.lds > GV1_LDS_MAX || p.nw == 0u ||
        p.nw > GV1_MAX_WAVES || p.nw % KS != 0u || (uint64_t)p.grid * p.nw < chunks ||
        p.act_dw != (M == 1u ? a.kb * 9u : 0u) || p.ks != (uint32_t)KS ||
        (KS == 1 ? p.cb != a.nbr : (uint64_t)p.cb * (KS - 1) >= a.nbr || (uint64_t)p.cb * KS < a.nbr)) {
        snprintf(err, errlen, "plan: lds %u region %u act %u waves %u grid %u parts %u of %u blocks for %llu rows",
                 p.lds, p.region_dw, p.act_dw, p.nw, p.grid, p.ks, p.cb, (unsigned long long)N);
        return 1;
    }
    if (!gv1_stage_cover(p.act_dw / 4u, p.nw, hits)) {  // the act_dw mod 4 last dwords: wave 0's lanes
        snprintf(err, errlen, "activation staging does not cover every group once");
        return 1;
    }
    std::vector<uint32_t> act_lds(gv1_act_region(p.act_dw) + 1u);
    memcpy(act_lds.data(), xq, 4u * (size_t)p.act_dw);
    if (p.act_dw > 0u && gv_uses_sum<F>())  // the workgroup's threads form the code sums
        for (uint32_t t = 0; t < 64u * p.nw; t++) gv1_act_prep(act_lds.data(), a.kb, t, 64u * p.nw);
    const GvActRaw act{act_lds.data()};                          // one activation row: from LDS
    const GvAct<false> gact{a.xq, nullptr, a.K, a.kb, a.xrow, a.M};  // several: from global memory
    Check chk{(uintptr_t)w, (uintptr_t)(w + N * a.row_bytes), 0, {0}};
    const HostSrc src{a.wbase, a.wlast, &chk};
    constexpr uint32_t IPB = GvItem<F>::IPB;
    const uint32_t S = (uint32_t)block_bytes(F);
    std::vector<uint32_t> lds(p.region_dw);
    std::vector<float> part((size_t)p.nw * MT);
    for (uint32_t b = 0; b < p.grid; b++) {
        std::fill(part.begin(), part.end(), 0.0f);
        for (uint32_t wave = 0; wave < p.nw; wave++) {
            const uint32_t cw = b * p.nw + wave;
            const uint32_t r = KS == 1 ? cw * (uint32_t)RW : cw / (uint32_t)KS;
            const uint32_t h = KS == 1 ? 0u : cw % (uint32_t)KS;
            if (r >= a.rows) continue;
            const GvChunk c = gv_chunk(a, r, h * a.cb);
            const uint32_t ng = c.g1 - c.g0 + 1u;
            const bool tail = 4u * c.g1 + 3u > a.wlast;
            const uint32_t nfull = tail ? ng - 1u : ng;
            if (4u * ng + 4u > p.region_dw || c.nb == 0u) {
                snprintf(err, errlen, "chunk of %u groups (%u blocks) past its region of %u dwords", ng, c.nb,
                         p.region_dw);
                return 1;
            }
            uint32_t active = 0u;  // chunk loads with at least one active lane
            for (uint32_t k = 0; 64u * k < ng; k++) active += 64u * k < nfull ? 1u : 0u;
            if ((nfull + 63u) / 64u != active) {
                snprintf(err, errlen, "wave waits on %u chunk loads, %u have an active lane", (nfull + 63u) / 64u,
                         active);
                return 1;
            }
            std::fill(lds.begin(), lds.end(), 0xA5A5A5A5u);
            for (uint32_t j = 0; j < nfull; j++) {  // lane j % 64 of load j / 64
                const uint32_t *g = a.wbase + 4u * (c.g0 + j);
                if (((uintptr_t)g & 15u) != 0u && chk.errors++ == 0)
                    snprintf(chk.msg, sizeof chk.msg, "16-byte load to LDS at %#lx not aligned", (unsigned long)g);
                uint32_t v[4];
                src.load<4>(4u * (c.g0 + j), v);
                for (int e = 0; e < 4; e++) lds[4u * j + (uint32_t)e] = v[e];
            }
            if (tail) {
                uint32_t v[1][4];
                src.load_stream4(a.wlast - 3u, v[0]);
                GvChunk one = c;
                one.g0 = c.g1;
                gv_put<1>(one, a.wlast, 0u, v, lds.data() + 4u * (ng - 1u));
            }
            for (uint32_t rr = 0; rr < c.rw; rr++) {
                const uint8_t *cb = (const uint8_t *)lds.data() + c.o0 + rr * a.row_bytes;
                const uint8_t *pb = w + (uint64_t)(c.r + rr) * a.row_bytes + (uint64_t)c.c0 * S;
                if (memcmp(cb, pb, (size_t)c.nb * S) != 0 && chk.errors++ == 0)
                    snprintf(chk.msg, sizeof chk.msg, "staged chunk of row %u differs from the payload", c.r + rr);
            }
            const Gv1Src<F> ls = gv_src<Gv1Src<F>>(lds.data(), 4u * (c.g1 - c.g0) + 3u);
            const uint32_t n = c.nb * IPB;
            static float acc[64][RW][MT];
            for (uint32_t lane = 0; lane < 64u; lane++) {
                for (int rr = 0; rr < RW; rr++)
                    for (int m = 0; m < MT; m++) acc[lane][rr][m] = 0.0f;
                if constexpr (MT == 1)
                    gv1_items1<F, RW>(ls, c, lane, a.row_bytes, n, act, tab, acc[lane]);
                else
                    gv_chunk_items<F, MT, RW>(ls, c, lane, a.M, a.row_bytes, gact, tab, acc[lane]);
            }
            for (uint32_t rr = 0; rr < c.rw; rr++)
                for (int m = 0; m < MT; m++) {
                    float v[64];
                    for (int l = 0; l < 64; l++) v[l] = acc[l][rr][m];
                    const float sum = dpp_sum63(v);
                    if (KS > 1)
                        part[(size_t)wave * MT + (size_t)m] = sum;
                    else if (m < (int)a.M)
                        a.y[(uint64_t)m * a.ldy + c.r + rr] = sum;
                }
        }
        if constexpr (KS > 1) {
            for (uint32_t wave = 0; wave < p.nw; wave += (uint32_t)KS) {
                const uint32_t r = (b * p.nw + wave) / (uint32_t)KS;
                if (r >= a.rows) continue;
                for (int m = 0; m < (int)a.M; m++) {
                    float t = part[(size_t)wave * MT + (size_t)m];
                    for (int j = 1; j < KS; j++) t += part[(size_t)(wave + (uint32_t)j) * MT + (size_t)m];
                    a.y[(uint64_t)m * a.ldy + r] = t;
                }
            }
        }
    }
    if (chk.errors) snprintf(err, errlen, "%s", chk.msg);
    return chk.errors;
}

template <int F, int MT, bool ALDS>
long run_gemv_alds(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y,
                   uint32_t resident, uint64_t max_rows, char *err, int errlen) {
    const uint64_t row_bytes = K / (uint64_t)nq::block_values(F) * (uint64_t)nq::block_bytes(F);
    switch (nq::gv_rows_per_chunk(row_bytes)) {
    case 4: return run_gemv_lds<F, MT, ALDS, 4>(w, N, K, xq, M, y, resident, max_rows, err, errlen);
    case 2: return run_gemv_lds<F, MT, ALDS, 2>(w, N, K, xq, M, y, resident, max_rows, err, errlen);
    default: return run_gemv_lds<F, MT, ALDS, 1>(w, N, K, xq, M, y, resident, max_rows, err, errlen);
    }
}

// The launcher's choice: with gv1_cus > 0, the single-round plan on a device
// of that many compute units, each holding min(gv1_per_cu, 160 KiB / (the
// workgroup's LDS)) workgroups (the tables' static LDS included); when it
// makes none, or with gv1_cus = 0, the chunk-loop kernel.  *rw_out: rows per
// chunk of the single-round launch (0 for the chunk loop), plus 256 times its
// parts per row.
template <int F, int MT>
long run_gemv(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y, uint32_t resident,
              uint64_t max_rows, uint32_t gv1_cus, uint32_t gv1_per_cu, uint32_t *rw_out, char *err, int errlen) {
    using namespace nq;
    *rw_out = 0u;
    if (gv1_cus > 0u) {
        const GvLaunch L{w, N, K, M, xq, y, gv1_cus};
        constexpr uint32_t stat = 8u * (uint32_t)TabSpec<F>::n8 + 4u * (uint32_t)TabSpec<F>::n4;
        const Gv1Plan p = gv1_plan(N, K / (uint64_t)block_values(F), (uint32_t)block_bytes(F), GvItem<F>::IPB, M,
                                   K, max_rows ? max_rows : gv_max_rows<F>(L), (uintptr_t)w, (uintptr_t)xq, gv1_cus,
                                   [&](uint32_t, uint32_t, uint32_t nw, uint32_t lds) {
                                       return gv1_emu_per_cu(gv1_per_cu, nw, lds + stat);
                                   });
        *rw_out = p.rw | p.ks << 8;
        if (p.ks == 2u) return run_gemv1<F, MT, 1, 2>(w, N, K, xq, M, y, p, err, errlen);
        if (p.rw == 1u) return run_gemv1<F, MT, 1, 1>(w, N, K, xq, M, y, p, err, errlen);
        if (p.rw == 2u) return run_gemv1<F, MT, 2, 1>(w, N, K, xq, M, y, p, err, errlen);
        if (p.rw == 3u) return run_gemv1<F, MT, 3, 1>(w, N, K, xq, M, y, p, err, errlen);
    }
    return nq::gv_act_in_lds(M, K) ? run_gemv_alds<F, MT, true>(w, N, K, xq, M, y, resident, max_rows, err, errlen)
                                   : run_gemv_alds<F, MT, false>(w, N, K, xq, M, y, resident, max_rows, err, errlen);
}

template <int F>
long run_gemv_m(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y, uint32_t res,
                uint64_t max_rows, uint32_t gv1_cus, uint32_t gv1_per_cu, uint32_t *rw_out, char *err, int errlen) {
    if (M <= 1) return run_gemv<F, 1>(w, N, K, xq, M, y, res, max_rows, gv1_cus, gv1_per_cu, rw_out, err, errlen);
    if (M <= 2) return run_gemv<F, 2>(w, N, K, xq, M, y, res, max_rows, gv1_cus, gv1_per_cu, rw_out, err, errlen);
    if (M <= 4) return run_gemv<F, 4>(w, N, K, xq, M, y, res, max_rows, gv1_cus, gv1_per_cu, rw_out, err, errlen);
    return run_gemv<F, 8>(w, N, K, xq, M, y, res, max_rows, gv1_cus, gv1_per_cu, rw_out, err, errlen);
}

// The 16 x 16 x 32 8-bit matrix instruction of one wave: lane l supplies row
// l mod 16 of A and column l mod 16 of B, code bytes k = 8 (l / 16) .. + 7 of
// each; lane l receives D[4 (l / 16) + e][l mod 16], e = 0..3.
void mfma_i8_16x16x32(const uint64_t (&A)[64], const uint64_t (&B)[64], int (&D)[64][4]) {
    int a[16][32], b[32][16];
    for (int l = 0; l < 64; l++)
        for (int t = 0; t < 8; t++) {
            a[l % 16][8 * (l / 16) + t] = (int)(int8_t)(uint8_t)(A[l] >> (8 * t));
            b[8 * (l / 16) + t][l % 16] = (int)(int8_t)(uint8_t)(B[l] >> (8 * t));
        }
    for (int l = 0; l < 64; l++)
        for (int e = 0; e < 4; e++) {
            const int i = 4 * (l / 16) + e, j = l % 16;
            int sum = 0;
            for (int k = 0; k < 32; k++) sum += a[i][k] * b[k][j];
            D[l][e] = sum;
        }
}

// The 16 x 16 x 4 binary32 matrix instruction of one wave (D = C + A B):
// lane l supplies A[l mod 16][l / 16] and B[l / 16][l mod 16] and holds
// C / D[4 (l / 16) + e][l mod 16]; the sum is formed here as a chain of
// fused multiply-adds in k order (the hardware's internal order may differ
// in the last bits; the results are judged by the criterion).
void mfma_f32_16x16x4(const float (&A)[64], const float (&B)[64], float (&C)[64][4]) {
    for (int l = 0; l < 64; l++)
        for (int e = 0; e < 4; e++) {
            const int i = 4 * (l / 16) + e, j = l % 16;
            float c = C[l][e];
            for (int k = 0; k < 4; k++) c = std::fma(A[16 * k + i], B[16 * k + j], c);
            C[l][e] = c;
        }
}

// Batched product on the matrix cores: the launcher's launches (max_rows /
// max_mrows > 0 override its weight-row and activation-row limits; cus > 0
// plans K splits for that many compute units, with a workspace), and per
// launch every workgroup of the grid as the kernel runs it: its tile and K
// split (each met exactly once), per K step the threads' staging into a
// poisoned LDS image (weight reads through a bounds-checked source), then per
// span and wave the lanes' operands, the matrix instruction and the lanes'
// scaling, and at the end the lanes' stores; then the partials' sum.
template <int F, int NI, int MJ, int SP>
long run_gemm_sh(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y,
                 uint64_t max_rows, uint64_t max_mrows, const nq::GmPlan &plan, char *err, int errlen) {
    using namespace nq;
    using Sh = GmShape<NI, MJ>;
    using G = GmFmt<F, Sh::BM, SP>;
    const GvLaunch L{w, N, K, M, xq, y, 0u};
    const uint64_t lim = max_rows ? max_rows : gm_max_rows<F>(L);
    const uint64_t mlim = max_mrows ? max_mrows : gm_max_mrows(K);
    const uint64_t row_bytes = K / (uint64_t)block_values(F) * (uint64_t)block_bytes(F);
    std::vector<uint64_t> t8(TabSpec<F>::n8 > 0 ? TabSpec<F>::n8 : 1);
    std::vector<uint32_t> t4(TabSpec<F>::n4 > 0 ? TabSpec<F>::n4 : 1);
    for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) gv_fill_tables<F>(t8.data(), t4.data(), tid);
    const Tab tab{t8.data(), t4.data(), nullptr, nullptr, 0xFFFFFFFFu, 1u};
    std::vector<uint32_t> lds(G::DW);
    static float acc[4][64][NI][MJ][4];
    static GmOps<NI, MJ> ops[64];
    static GmI<F, NI, MJ> I[64];
    long errors = 0;
    if (plan.sp != G::SP) {
        snprintf(err, errlen, "K step of %u spans, kernel built for %u", plan.sp, G::SP);
        return 1;
    }
    const GmWsLayout wl = gm_ws_layout(F, plan, N, K, M);
    std::vector<uint8_t> wsbuf(wl.total + 256, 0xA5);
    uint8_t *wsp = wsbuf.data() + (256 - (uintptr_t)wsbuf.data() % 256) % 256;
    float *part = (float *)wsp;
    float *out = plan.nsplit > 1 ? part : y;
    uint8_t *canon = plan.rewrite_once ? wsp : nullptr;
    if (canon) {  // the rewrite launches, one item per thread
        for (uint64_t r0 = 0; r0 < N;) {
            const uint64_t rows = N - r0 < lim ? N - r0 : lim;
            const GmArgs a = gm_args<F>(L, r0, rows, 0, 1, plan, out, canon, &wl);
            Check chk{(uintptr_t)(w + r0 * row_bytes), (uintptr_t)(w + (r0 + rows) * row_bytes), 0, {0}};
            const HostSrc src{a.wbase, a.wlast, &chk};
            const uint64_t blocks = (gm_rewrite_items(a.rows, a.kspans) + WG - 1) / WG;
            for (uint64_t g = 0; g < blocks * WG; g++)
                gm_rewrite_item<F>(a, src, tab, g, (uint32_t *)(canon + wl.codes + r0 * K),
                                   (float *)(canon + wl.scales) + r0, (float *)(canon + wl.offsets) + r0);
            if (chk.errors) {
                if (errors == 0) snprintf(err, errlen, "rewrite: %s", chk.msg);
                errors += chk.errors;
            }
            r0 += rows;
        }
    }
    for (uint64_t m0 = 0; m0 < M; m0 += mlim) {
        const uint64_t mrows = M - m0 < mlim ? M - m0 : mlim;
        for (uint64_t r0 = 0; r0 < N;) {
            const uint64_t rows = N - r0 < lim ? N - r0 : lim;
            const GmArgs a = gm_args<F>(L, r0, rows, m0, mrows, plan, out, canon, &wl);
            Check chk{(uintptr_t)(w + r0 * row_bytes), (uintptr_t)(w + (r0 + rows) * row_bytes), 0, {0}};
            const HostSrc src{a.wbase, a.wlast, &chk};
            const uint32_t grid = gm_grid(a);
            const uint32_t nt = (uint32_t)((rows + GM_BN - 1) / GM_BN);
            if ((uint64_t)grid != (uint64_t)nt * a.mt * a.nsplit) {
                snprintf(err, errlen, "grid %u for %u x %u tiles x %u splits", grid, nt, a.mt, a.nsplit);
                return 1;
            }
            std::vector<char> seen(grid, 0);
            for (uint32_t id = 0; id < grid; id++) {
                uint32_t n0, mt0, ks;
                gm_tile(a, id, &n0, &mt0, &ks);
                if (a.bm != G::BM) {
                    snprintf(err, errlen, "tile height %u, kernel built for %u", a.bm, G::BM);
                    return 1;
                }
                const uint64_t tile = ((uint64_t)(n0 / GM_BN) * a.mt + mt0 / a.bm) * a.nsplit + ks;
                if (n0 % GM_BN || mt0 % a.bm || ks >= a.nsplit || tile >= grid || seen[tile]++) {
                    snprintf(err, errlen, "workgroup %u: tile (%u, %u, %u) out of range or met twice", id, n0, mt0,
                             ks);
                    return 1;
                }
                for (auto &wv : acc)
                    for (auto &ln : wv)
                        for (auto &i4 : ln)
                            for (auto &j2 : i4)
                                for (float &v : j2) v = 0.0f;
                const uint32_t tb = ks * a.sps * G::SP, te0 = tb + a.sps * G::SP,
                               te = te0 < a.kspans ? te0 : a.kspans;
                for (uint32_t t0 = tb; t0 < te; t0 += G::SP) {
                    std::fill(lds.begin(), lds.end(), 0xA5A5A5A5u);
                    for (uint32_t tid = 0; tid < (uint32_t)WG; tid++) {
                        if (a.cw)
                            gm_stage_wc<F, SP>(a, n0, t0, tid, lds.data());
                        else
                            gm_stage_w<F, SP>(a, src, tab, n0, t0, tid, lds.data());
                    }
                    for (uint32_t tid = 0; tid < (uint32_t)WG; tid++)
                        gm_stage_x<F, Sh::BM, SP>(a, mt0, t0, tid, lds.data());
                    const uint32_t nsp = te - t0 < G::SP ? te - t0 : G::SP;
                    for (uint32_t sp = 0; sp < nsp; sp++)
                        for (uint32_t wv = 0; wv < 4u; wv++) {
                            for (uint32_t lane = 0; lane < 64u; lane++)
                                gm_ops<F, NI, MJ, SP>(lds.data(), wv, lane, sp, ops[lane]);
                            for (uint32_t h = 0; h < G::NH; h++)
                                for (int j = 0; j < MJ; j++)
                                    for (int i = 0; i < NI; i++) {
                                        uint64_t A[64], B[64];
                                        int D[64][4];
                                        for (uint32_t l = 0; l < 64u; l++) {
                                            A[l] = ops[l].A[i];
                                            B[l] = gm_half<F>(ops[l].B[j], l, h);
                                        }
                                        mfma_i8_16x16x32(A, B, D);
                                        for (int l = 0; l < 64; l++)
                                            for (int e = 0; e < 4; e++) I[l].v[h][i][j][e] = D[l][e];
                                    }
                            for (uint32_t lane = 0; lane < 64u; lane++)
                                gm_epi<F, NI, MJ, SP>(lds.data(), wv, lane, sp, I[lane], acc[wv][lane]);
                        }
                    if constexpr (G::AFF) {
                        const uint32_t nk = nsp * G::NH;
                        for (uint32_t q = 0; 4u * q < nk; q++)
                            for (uint32_t wv = 0; wv < 4u; wv++) {
                                float Al[64][NI], Bl[64][MJ];
                                for (uint32_t lane = 0; lane < 64u; lane++) {
                                    float a4[NI], b2[MJ];
                                    gm_offsets_ops<F, NI, MJ, SP>(lds.data(), wv, lane, q, nk, a4, b2);
                                    for (int i = 0; i < NI; i++) Al[lane][i] = a4[i];
                                    for (int j = 0; j < MJ; j++) Bl[lane][j] = b2[j];
                                }
                                for (int i = 0; i < NI; i++)
                                    for (int j = 0; j < MJ; j++) {
                                        float A[64], B[64], C[64][4];
                                        for (int l = 0; l < 64; l++) {
                                            A[l] = Al[l][i];
                                            B[l] = Bl[l][j];
                                            for (int e = 0; e < 4; e++) C[l][e] = acc[wv][l][i][j][e];
                                        }
                                        mfma_f32_16x16x4(A, B, C);
                                        for (int l = 0; l < 64; l++)
                                            for (int e = 0; e < 4; e++) acc[wv][l][i][j][e] = C[l][e];
                                    }
                            }
                    }
                }
                for (uint32_t wv = 0; wv < 4u; wv++)
                    for (uint32_t lane = 0; lane < 64u; lane++)
                        gm_store<NI, MJ>(a, n0, mt0, ks, wv, lane, acc[wv][lane]);
            }
            if (chk.errors) {
                if (errors == 0) snprintf(err, errlen, "%s", chk.msg);
                errors += chk.errors;
            }
            r0 += rows;
        }
    }
    if (plan.nsplit > 1) {
        const uint64_t n = M * N;
        for (uint64_t i = 0; i < n; i++) {
            float v = part[i];
            for (uint32_t sidx = 1; sidx < plan.nsplit; sidx++) v = v + part[(uint64_t)sidx * n + i];
            y[i] = v;
        }
    }
    return errors;
}

// The launcher's plan and kernel for M activation rows: cus > 0 plans for a
// device of that many compute units with the workspace the plan asks for;
// 0: no workspace (neither split nor per-call rewrite) and 8-span K steps.
// *plan_out: nsplit, bit 16 the per-call rewrite, bit 17 4-span K steps.
template <int F>
long run_gemm(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y, uint64_t max_rows,
              uint64_t max_mrows, uint32_t cus, uint32_t *plan_out, char *err, int errlen) {
    using namespace nq;
    GmPlan p = gm_plan(F, N, K, M, cus);
    if (cus == 0) p = gm_plan_plain(GmPlan{1u, 0u, false, GM_SP}, K);
    *plan_out = p.nsplit | (p.rewrite_once ? 1u << 16 : 0u) | (p.sp == 4u ? 1u << 17 : 0u);
    const uint32_t bm = gm_bm(M);
    if (bm == 64u && p.sp == 4u) return run_gemm_sh<F, 4, 2, 4>(w, N, K, xq, M, y, max_rows, max_mrows, p, err, errlen);
    if (bm == 64u) return run_gemm_sh<F, 4, 2, 8>(w, N, K, xq, M, y, max_rows, max_mrows, p, err, errlen);
    if (bm == 32u) return run_gemm_sh<F, 4, 1, 8>(w, N, K, xq, M, y, max_rows, max_mrows, p, err, errlen);
    return run_gemm_sh<F, 2, 1, 8>(w, N, K, xq, M, y, max_rows, max_mrows, p, err, errlen);
}

}  // namespace

using EmuRun = long (*)(int ot, const uint8_t *payload, uint64_t nbytes, uint64_t nblocks, void *out,
                       uint32_t max_wgs, uint64_t chunk, int force_upt, uint32_t ndiv, char *err, int errlen);
extern EmuRun nq_emu_table[nq::NUM_FORMATS];
using EmuGemv = long (*)(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y,
                         uint32_t resident, uint64_t max_rows, uint32_t gv1_cus, uint32_t gv1_per_cu,
                         uint32_t *rw_out, char *err, int errlen);
extern EmuGemv nq_emu_gemv_table[nq::NUM_FORMATS];
using EmuGemm = long (*)(const uint8_t *w, uint64_t N, uint64_t K, const uint8_t *xq, uint64_t M, float *y,
                         uint64_t max_rows, uint64_t max_mrows, uint32_t cus, uint32_t *nsplit, char *err,
                         int errlen);
extern EmuGemm nq_emu_gemm_table[nq::NUM_FORMATS];
using EmuMany = long (*)(int ot, const nq::ManyItem *items, int n, uint32_t resident, uint64_t chunk, int *launches,
                         int *upt_mask, char *err, int errlen);
extern EmuMany nq_emu_many_table[nq::NUM_FORMATS];

#if defined(NQ_EMU_PART)
namespace {
template <int F>
void reg() {
    if constexpr (F % NQ_EMU_PARTS == NQ_EMU_PART) {
        nq_emu_table[F] = &run_ot<F>;
        nq_emu_many_table[F] = &run_many_ot<F>;
        if constexpr (F != nq::NVFP4_DIV) nq_emu_gemv_table[F] = &run_gemv_m<F>;
        if constexpr (nq::GmFmt<F>::OK) nq_emu_gemm_table[F] = &run_gemm<F>;
    }
}
struct Register {
    Register() {
        using namespace nq;
        reg<Q4_0>(); reg<Q4_1>(); reg<Q5_0>(); reg<Q5_1>(); reg<Q8_0>(); reg<Q8_1>(); reg<Q2_K>(); reg<Q3_K>();
        reg<Q4_K>(); reg<Q5_K>(); reg<Q6_K>(); reg<Q8_K>(); reg<IQ2_XXS>(); reg<IQ2_XS>(); reg<IQ3_XXS>();
        reg<IQ1_S>(); reg<IQ4_NL>(); reg<IQ3_S>(); reg<IQ2_S>(); reg<IQ4_XS>(); reg<IQ1_M>(); reg<TQ1_0>();
        reg<TQ2_0>(); reg<MXFP4>(); reg<NVFP4_GGUF>(); reg<Q1_0>(); reg<Q2_0>(); reg<NVFP4_DIV>();
    }
} registered;
}  // namespace
#else
EmuRun nq_emu_table[nq::NUM_FORMATS];
EmuGemv nq_emu_gemv_table[nq::NUM_FORMATS];
EmuGemm nq_emu_gemm_table[nq::NUM_FORMATS];
EmuMany nq_emu_many_table[nq::NUM_FORMATS];

// Many-tensor decode of n tensors of one format (payload, nbytes, blocks and
// output of each; all outputs 16-byte aligned or none), through the
// launcher's packing (chunk: blocks per launch chunk, 0 for the library's)
// and the kernel's tile search; returns out-of-payload reads and mapping
// errors (0 on success), or -1 for a bad format.
extern "C" __attribute__((visibility("default"))) long nq_emu_decode_many(int fmt, int ot, int n,
                                                                         const uint8_t *const *payloads,
                                                                         const uint64_t *nbytes,
                                                                         const uint64_t *nblocks, void *const *outs,
                                                                         uint32_t resident, uint64_t chunk,
                                                                         int *launches, int *upt_mask, char *err,
                                                                         int errlen) {
    if (fmt < 0 || fmt >= nq::NUM_FORMATS || !nq_emu_many_table[fmt] || n < 0) return -1;
    std::vector<nq::ManyItem> items((size_t)n);
    for (int i = 0; i < n; i++) items[(size_t)i] = nq::ManyItem{payloads[i], nbytes[i], nblocks[i], outs[i]};
    return nq_emu_many_table[fmt](ot, items.data(), n, resident, chunk, launches, upt_mask, err, errlen);
}

// Batched product on the matrix cores through the kernel's lane code;
// returns out-of-payload weight reads (0 on success), or -1 for a format
// without a span rewrite.
extern "C" __attribute__((visibility("default"))) long nq_emu_gemm_q8_1(int fmt, const uint8_t *w, uint64_t N,
                                                                       uint64_t K, const uint8_t *xq, uint64_t M,
                                                                       float *y, uint64_t max_rows,
                                                                       uint64_t max_mrows, uint32_t cus,
                                                                       uint32_t *nsplit, char *err, int errlen) {
    if (fmt < 0 || fmt >= nq::NUM_FORMATS || !nq_emu_gemm_table[fmt]) return -1;
    return nq_emu_gemm_table[fmt](w, N, K, xq, M, y, max_rows, max_mrows, cus, nsplit, err, errlen);
}

// The batched product's plan on a device of `cus` compute units, as the
// launcher makes it: out = {K splits, steps per split, spans per step,
// weight rewritten once, tile height, workspace bytes, and the plan without
// a workspace: K splits, steps per split, spans per step}.
extern "C" __attribute__((visibility("default"))) void nq_emu_gemm_plan(int fmt, uint64_t N, uint64_t K, uint64_t M,
                                                                       uint32_t cus, uint64_t *out) {
    const nq::GmPlan p = nq::gm_plan(fmt, N, K, M, cus), q = nq::gm_plan_plain(p, K);
    out[0] = p.nsplit;
    out[1] = p.sps;
    out[2] = p.sp;
    out[3] = p.rewrite_once ? 1u : 0u;
    out[4] = nq::gm_bm(M);
    out[5] = nq::gm_ws_layout(fmt, p, N, K, M).total;
    out[6] = q.nsplit;
    out[7] = q.sps;
    out[8] = q.sp;
}

// The single-round product plan, as run_gemv models the device (gv1_cus
// compute units, at most gv1_per_cu workgroups each, 160 KiB of LDS), for
// weight bytes starting `w_mis` bytes past a 16-byte boundary: out = {rows
// per chunk (0: none), region dwords, LDS bytes, workgroups}.
template <int F>
void gv1_plan_of(uint64_t N, uint64_t K, uint64_t M, uint32_t w_mis, uint32_t cus, uint32_t per_cu, uint64_t *out) {
    using namespace nq;
    constexpr uint32_t stat = 8u * (uint32_t)TabSpec<F>::n8 + 4u * (uint32_t)TabSpec<F>::n4;
    const GvLaunch L{nullptr, N, K, M, nullptr, nullptr, cus};
    const Gv1Plan p = gv1_plan(N, K / (uint64_t)block_values(F), (uint32_t)block_bytes(F), GvItem<F>::IPB, M, K,
                               gv_max_rows<F>(L), (uintptr_t)(4096u + w_mis), (uintptr_t)4096u, cus,
                               [&](uint32_t, uint32_t, uint32_t nw, uint32_t lds) {
                                   return gv1_emu_per_cu(per_cu, nw, lds + stat);
                               });
    out[0] = p.rw;
    out[1] = p.region_dw;
    out[2] = p.lds;
    out[3] = p.grid;
    out[4] = p.ks;
    out[5] = p.cb;
    out[6] = p.nw;
    out[7] = p.act_dw;
}

extern "C" __attribute__((visibility("default"))) int nq_emu_gemv1_plan(int fmt, uint64_t N, uint64_t K, uint64_t M,
                                                                       uint32_t w_mis, uint32_t cus,
                                                                       uint32_t per_cu, uint64_t *out) {
    using namespace nq;
    switch (fmt) {
#define NQ_GV1_CASE(X) \
    case X: gv1_plan_of<X>(N, K, M, w_mis, cus, per_cu, out); return 0;
    NQ_GV1_CASE(Q4_0) NQ_GV1_CASE(Q4_1) NQ_GV1_CASE(Q5_0) NQ_GV1_CASE(Q5_1) NQ_GV1_CASE(Q8_0) NQ_GV1_CASE(Q8_1)
    NQ_GV1_CASE(Q2_K) NQ_GV1_CASE(Q3_K) NQ_GV1_CASE(Q4_K) NQ_GV1_CASE(Q5_K) NQ_GV1_CASE(Q6_K) NQ_GV1_CASE(Q8_K)
    NQ_GV1_CASE(IQ2_XXS) NQ_GV1_CASE(IQ2_XS) NQ_GV1_CASE(IQ3_XXS) NQ_GV1_CASE(IQ1_S) NQ_GV1_CASE(IQ4_NL)
    NQ_GV1_CASE(IQ3_S) NQ_GV1_CASE(IQ2_S) NQ_GV1_CASE(IQ4_XS) NQ_GV1_CASE(IQ1_M) NQ_GV1_CASE(TQ1_0)
    NQ_GV1_CASE(TQ2_0) NQ_GV1_CASE(MXFP4) NQ_GV1_CASE(NVFP4_GGUF) NQ_GV1_CASE(Q1_0) NQ_GV1_CASE(Q2_0)
#undef NQ_GV1_CASE
    default: return -1;
    }
}

// Product with q8_1 activations through the kernel's lane code (the
// single-round kernel when gv1_cus > 0 and its plan exists, see run_gemv);
// returns out-of-payload weight reads (0 on success), or -1 for a format
// without one.
extern "C" __attribute__((visibility("default"))) long nq_emu_gemv_q8_1(int fmt, const uint8_t *w, uint64_t N,
                                                                       uint64_t K, const uint8_t *xq, uint64_t M,
                                                                       float *y, uint32_t resident,
                                                                       uint64_t max_rows, uint32_t gv1_cus,
                                                                       uint32_t gv1_per_cu, uint32_t *rw_out,
                                                                       char *err, int errlen) {
    if (fmt < 0 || fmt >= nq::NUM_FORMATS || !nq_emu_gemv_table[fmt]) return -1;
    return nq_emu_gemv_table[fmt](w, N, K, xq, M, y, resident, max_rows, gv1_cus, gv1_per_cu, rw_out, err, errlen);
}

// Returns the number of out-of-payload reads (0 on success), or -1 for a bad format.
// ndiv: "nvfp4" divisor words after the blocks (stacked sources), 1 otherwise.
extern "C" __attribute__((visibility("default"))) long nq_emu_decode(int fmt, int ot, const uint8_t *payload,
                                                                    uint64_t nbytes, uint64_t nblocks, void *out,
                                                                    uint32_t max_wgs, uint64_t chunk_blocks,
                                                                    int force_upt, uint32_t ndiv, char *err,
                                                                    int errlen) {
    if (fmt < 0 || fmt >= nq::NUM_FORMATS || !nq_emu_table[fmt]) return -1;
    return nq_emu_table[fmt](ot, payload, nbytes, nblocks, out, max_wgs, chunk_blocks, force_upt,
                             ndiv < 1 ? 1 : ndiv, err, errlen);
}

// The "nvfp4" quotient table for each of n divisor words, built as the
// kernels build it (nvfp4_table_quad, four entries per thread) and entry by
// entry (nvfp4_table_entry, one division each): 1024 words per divisor in
// `quad` and `direct`.
extern "C" __attribute__((visibility("default"))) void nq_emu_nvfp4_tables(const uint32_t *dw_bits, long n,
                                                                          uint32_t *quad, uint32_t *direct) {
    for (long i = 0; i < n; i++) {
        const float dw = nq::bits_f32(dw_bits[i]);
        uint32_t *q = quad + 1024 * i, *d = direct + 1024 * i;
        for (uint32_t k = 0; k < 256; k++) {
            uint32_t e[4], code[4];
            nq::nvfp4_table_quad(k >> 1, k & 1u, dw, e, code);
            for (int j = 0; j < 4; j++) q[8u * (k >> 1) + code[j]] = e[j];
        }
        for (uint32_t k = 0; k < 1024; k++) d[k] = nq::nvfp4_table_entry(k, dw);
    }
}

// Whole blocks per staged tile of format fmt at `upt` units per thread, for
// tests that place tile boundaries.
extern "C" __attribute__((visibility("default"))) long nq_emu_tile_blocks(int fmt, int upt) {
    using namespace nq;
    switch (fmt) {
#define C(X) \
    case X: return tile_blocks<X>(upt);
        C(Q4_0) C(Q4_1) C(Q5_0) C(Q5_1) C(Q8_0) C(Q8_1) C(Q2_K) C(Q3_K) C(Q4_K) C(Q5_K) C(Q6_K) C(Q8_K)
        C(IQ2_XXS) C(IQ2_XS) C(IQ3_XXS) C(IQ1_S) C(IQ4_NL) C(IQ3_S) C(IQ2_S) C(IQ4_XS) C(IQ1_M)
        C(TQ1_0) C(TQ2_0) C(MXFP4) C(NVFP4_GGUF) C(Q1_0) C(Q2_0) C(NVFP4_DIV)
#undef C
    default: return -1;
    }
}

// The launcher's choice of units per thread for a launch of `nunits` units
// of format fmt.
extern "C" __attribute__((visibility("default"))) int nq_emu_choose_upt(int fmt, uint64_t nunits, uint32_t resident) {
    using namespace nq;
    switch (fmt) {
#define C(X) \
    case X: return choose_upt<X>(nunits, resident);
        C(Q4_0) C(Q4_1) C(Q5_0) C(Q5_1) C(Q8_0) C(Q8_1) C(Q2_K) C(Q3_K) C(Q4_K) C(Q5_K) C(Q6_K) C(Q8_K)
        C(IQ2_XXS) C(IQ2_XS) C(IQ3_XXS) C(IQ1_S) C(IQ4_NL) C(IQ3_S) C(IQ2_S) C(IQ4_XS) C(IQ1_M)
        C(TQ1_0) C(TQ2_0) C(MXFP4) C(NVFP4_GGUF) C(Q1_0) C(Q2_0) C(NVFP4_DIV)
#undef C
    default: return -1;
    }
}

namespace {

// Row-scaled FP8: the launcher's chunk loop (chunk values per launch) and
// every thread of every launch, reading through bounds-checked sources.
template <int SK, int OT>
long run_fp8_row(const uint8_t *payload, uint64_t N, uint64_t K, void *out, uint64_t chunk, char *err, int errlen) {
    using namespace nq;
    constexpr uint64_t OSZ = OT == 0 ? 4 : OT == 3 ? 8 : 2;
    const F8Launch L{payload, N, K, out};
    const uint64_t total = N * K;
    long errors = 0;
    for (uint64_t E0 = 0; E0 < total; E0 += chunk) {
        uint32_t grid;
        const F8Args a = f8_chunk_args<OT>(L, E0, &grid, chunk);
        const uint64_t n = a.n, r0 = E0 / K, r1 = (E0 + n - 1) / K;
        Check cc{(uintptr_t)(payload + E0), (uintptr_t)(payload + E0 + n), 0, {0}};
        Check cs{(uintptr_t)(payload + total + 2 * r0), (uintptr_t)(payload + total + 2 * (r1 + 1)), 0, {0}};
        const HostSrc csrc{a.cbase, a.clast, &cc}, ssrc{a.sbase, a.slast, &cs};
        const bool vec = (((uintptr_t)out + E0 * OSZ) & 15) == 0;
        // per workgroup: if its last wave block is fast, every wave stages its
        // blocks (all lanes), then decodes them; otherwise unit by unit.  LDS
        // words are poisoned beforehand.
        std::vector<uint32_t> wbuf(256);
        for (uint32_t b = 0; b < grid; b++) {
            const bool fast = f8_fast_block(a, f8_wave_block(b, 3u, F8_NB - 1));
            for (uint32_t wave = 0; wave < 4u; wave++)
                for (int k = 0; k < F8_NB; k++) {
                    const uint32_t q = f8_wave_block(b, wave, k);
                    if (fast) {
                        std::fill(wbuf.begin(), wbuf.end(), 0xA5A5A5A5u);
                        for (uint32_t lane = 0; lane < 64u; lane++) {
                            uint32_t w[4];
                            fp8row_stage_load(csrc, q, lane, w);
                            for (int j = 0; j < 4; j++) wbuf[4u * lane + j] = w[j];
                        }
                        for (uint32_t lane = 0; lane < 64u; lane++) {
                            if (vec)
                                fp8row_wave_decode<SK, OT, true>(ssrc, a, q, lane, wbuf.data());
                            else
                                fp8row_wave_decode<SK, OT, false>(ssrc, a, q, lane, wbuf.data());
                        }
                    } else {
                        for (uint32_t lane = 0; lane < 64u; lane++)
                            for (uint32_t h = 0; h < 2u; h++) {
                                if (vec)
                                    fp8row_unit_direct<SK, OT, true>(csrc, ssrc, a, 128u * q + 64u * h + lane);
                                else
                                    fp8row_unit_direct<SK, OT, false>(csrc, ssrc, a, 128u * q + 64u * h + lane);
                            }
                    }
                }
        }
        for (Check *c : {&cc, &cs})
            if (c->errors) {
                if (errors == 0) snprintf(err, errlen, "%s", c->msg);
                errors += c->errors;
            }
    }
    return errors;
}

template <int SK>
long run_fp8_row_ot(int ot, const uint8_t *p, uint64_t N, uint64_t K, void *out, uint64_t chunk, char *err,
                    int errlen) {
    switch (ot) {
    case 0: return run_fp8_row<SK, 0>(p, N, K, out, chunk, err, errlen);
    case 1: return run_fp8_row<SK, 1>(p, N, K, out, chunk, err, errlen);
    case 2: return run_fp8_row<SK, 2>(p, N, K, out, chunk, err, errlen);
    default: return run_fp8_row<SK, 3>(p, N, K, out, chunk, err, errlen);
    }
}

}  // namespace

// Row-scaled FP8 through the kernel's per-thread code; returns out-of-bounds
// reads (0 on success).  chunk: values per launch (0: the launcher's).
extern "C" __attribute__((visibility("default"))) long nq_emu_fp8_row(int kind, int ot, const uint8_t *payload,
                                                                     uint64_t N, uint64_t K, void *out,
                                                                     uint64_t chunk, char *err, int errlen) {
    if (chunk == 0) chunk = nq::F8_CHUNK;
    return kind == 0 ? run_fp8_row_ot<0>(ot, payload, N, K, out, chunk, err, errlen)
                     : run_fp8_row_ot<1>(ot, payload, N, K, out, chunk, err, errlen);
}
// The multiply-shift division of the row-scaled FP8 and encoder kernels:
// floor(n / d) as computed from div_magic, for the test against plain
// division.
extern "C" __attribute__((visibility("default"))) uint32_t nq_emu_f8_div(uint32_t n, uint32_t d) {
    uint32_t m, sh;
    nq::div_magic(d, &m, &sh);
    return (uint32_t)(((uint64_t)n * m) >> sh);
}
// The K-quant sub-scale and min pair of a 64-value product item (g < 4)
// from the 12 packed scale bytes h[0..2], as the word [sc(2g), sc(2g+1),
// m(2g), m(2g+1)].
extern "C" __attribute__((visibility("default"))) uint32_t nq_emu_kq_scale_min_pair(uint32_t h0, uint32_t h1,
                                                                                   uint32_t h2, uint32_t g) {
    const uint32_t h[3] = {h0, h1, h2};
    return nq::kq_scale_min_pair(h, g);
}
namespace {

// Source reader of the encoder emulation: element reads and 16-byte reads,
// each checked against the launch's source elements [0, count).
template <int ESZ>
struct GqHostSrc {
    const void *x;
    uint64_t count;
    Check *chk;
    void check(uint64_t i, uint64_t n) const {
        if (i + n > count && chk->errors++ == 0)
            snprintf(chk->msg, sizeof chk->msg, "source elements %llu..%llu past %llu", (unsigned long long)i,
                     (unsigned long long)(i + n), (unsigned long long)count);
    }
    template <int IN>
    float one(uint64_t i) const {
        check(i, 1);
        return nq::gq_word_to_f32<IN>(x, i);
    }
    template <int IN>
    void span(uint64_t i, float (&v)[nq::gq_vpl<IN>()]) const {
        check(i, nq::gq_vpl<IN>());
        if (((uintptr_t)x + i * ESZ) % 16 != 0 && chk->errors++ == 0)
            snprintf(chk->msg, sizeof chk->msg, "16-byte source load at element %llu is misaligned",
                     (unsigned long long)i);
        nq::GqDevSrc{x}.span<IN>(i, v);
    }
};

// The encoder launcher's decisions and chunks, and for every group of every
// launch its lanes' phases: loads, the amax exchange, the encode and stores.
template <int S, int IN>
long run_gq(const void *x, uint64_t N, uint64_t K, int8_t *codes, uint16_t *scales, uint32_t *status, char *err,
            int errlen) {
    using namespace nq;
    constexpr uint64_t ESZ = IN == 0 ? 4 : IN == 3 ? 8 : 2;
    constexpr int GQ_VPL = gq_vpl<IN>();
    constexpr uint32_t G = (uint32_t)GQ[S].G, LPG = G / (uint32_t)GQ_VPL;
    const bool vin = (uintptr_t)x % 16 == 0 && (K * ESZ) % 16 == 0;
    const bool vout = (uintptr_t)codes % 4 == 0 && K % 4 == 0;
    const GqLaunch L{x, codes, scales, status, N, K};
    *status = 0u;
    long errors = 0;
    for (uint64_t r0 = 0; r0 < N;) {
        uint64_t rows;
        uint32_t grid;
        const GqArgs a = gq_chunk_args<S, IN>(L, r0, &rows, &grid);
        if ((uint64_t)grid * WG < (uint64_t)a.ngroups * LPG) {
            snprintf(err, errlen, "grid %u too small", grid);
            return 1;
        }
        Check chk{0, 0, 0, {0}};
        const GqHostSrc<(int)ESZ> src{a.x, rows * K, &chk};
        for (uint32_t g = 0; g < a.ngroups; g++) {
            float v[LPG][GQ_VPL];
            uint64_t off[LPG];
            uint32_t cnt[LPG];
            uint32_t mag = 0u;
            for (uint32_t j = 0; j < LPG; j++) {
                cnt[j] = gq_chunk<GQ_VPL>(a, (int)G, g, j, &off[j]);
                const uint32_t m = vin ? gq_load<IN, true>(src, off[j], cnt[j], v[j])
                                       : gq_load<IN, false>(src, off[j], cnt[j], v[j]);
                mag = gq_umax(mag, m);
            }
            for (uint32_t j = 0; j < LPG; j++) {
                uint32_t s16 = 0;
                uint32_t q[GQ_VPL / 4];
                const uint32_t st = mag >= GQ_NONFINITE ? 1u : gq_encode<S>(bits_f32(mag), v[j], &s16, q);
                if (st) {
                    *status |= st;
                    continue;
                }
                if (vout)
                    gq_store<true, GQ_VPL>(a, off[j], cnt[j], q, g, j, s16);
                else
                    gq_store<false, GQ_VPL>(a, off[j], cnt[j], q, g, j, s16);
            }
        }
        if (chk.errors) {
            if (errors == 0) snprintf(err, errlen, "%s", chk.msg);
            errors += chk.errors;
        }
        r0 += rows;
    }
    return errors;
}

template <int S>
long run_gq_in(int in, const void *x, uint64_t N, uint64_t K, int8_t *c, uint16_t *sc, uint32_t *st, char *err,
               int errlen) {
    switch (in) {
    case 0: return run_gq<S, 0>(x, N, K, c, sc, st, err, errlen);
    case 1: return run_gq<S, 1>(x, N, K, c, sc, st, err, errlen);
    case 2: return run_gq<S, 2>(x, N, K, c, sc, st, err, errlen);
    default: return run_gq<S, 3>(x, N, K, c, sc, st, err, errlen);
    }
}

}  // namespace

// grouped_absmax through the encoder's own lane code; returns out-of-bounds
// or misaligned source reads (0 on success) and stores the status bits.
extern "C" __attribute__((visibility("default"))) long nq_emu_grouped_absmax(int scheme, int in, const void *x,
                                                                            uint64_t N, uint64_t K, int8_t *codes,
                                                                            uint16_t *scales, uint32_t *status,
                                                                            char *err, int errlen) {
    switch (scheme) {
    case 0: return run_gq_in<0>(in, x, N, K, codes, scales, status, err, errlen);
    case 1: return run_gq_in<1>(in, x, N, K, codes, scales, status, err, errlen);
    case 2: return run_gq_in<2>(in, x, N, K, codes, scales, status, err, errlen);
    default: return run_gq_in<3>(in, x, N, K, codes, scales, status, err, errlen);
    }
}
namespace {

// q8_1 quantizer: the launcher's chunks and, per block, its lanes' phases:
// loads (bounds-checked), the amax / failure exchange, the encode, the code
// sum exchange and the stores.
template <int IN>
long run_q81(const void *x, uint64_t nblocks, uint32_t *blocks, uint32_t *status, uint64_t chunk, char *err,
             int errlen) {
    using namespace nq;
    constexpr uint64_t ESZ = IN == 0 ? 4 : IN == 3 ? 8 : 2;
    constexpr int VPL = gq_vpl<IN>();
    constexpr uint32_t LPB = q81_lanes<IN>();
    const bool vin = (uintptr_t)x % 16 == 0;
    *status = 0u;
    long errors = 0;
    for (uint64_t b0 = 0; b0 < nblocks; b0 += chunk) {
        Q81Args a;
        a.x = (const uint8_t *)x + b0 * 32 * ESZ;
        a.blocks = blocks + b0 * 9;
        a.status = status;
        a.nblocks = (uint32_t)(nblocks - b0 < chunk ? nblocks - b0 : chunk);
        Check chk{0, 0, 0, {0}};
        const GqHostSrc<(int)ESZ> src{a.x, (uint64_t)a.nblocks * 32u, &chk};
        for (uint32_t b = 0; b < a.nblocks; b++) {
            float v[LPB][VPL];
            uint32_t mag = 0u;
            for (uint32_t j = 0; j < LPB; j++) {
                const uint64_t o = (uint64_t)b * 32u + j * (uint32_t)VPL;
                const uint32_t m = vin ? gq_load<IN, true>(src, o, (uint32_t)VPL, v[j])
                                       : gq_load<IN, false>(src, o, (uint32_t)VPL, v[j]);
                mag = gq_umax(mag, m);
            }
            uint32_t q[LPB][VPL / 4];
            uint32_t d16[LPB], st[LPB];
            int sum = 0;
            for (uint32_t j = 0; j < LPB; j++) {
                st[j] = q81_encode<VPL>(mag, v[j], &d16[j], q[j]);
                sum += q81_sum<VPL>(q[j]);
            }
            for (uint32_t j = 0; j < LPB; j++) {
                const uint32_t bits = q81_store<VPL>(a, b, j, q[j], d16[j], sum, st[j]);
                if (j == 0u) *status |= bits;
            }
        }
        if (chk.errors) {
            if (errors == 0) snprintf(err, errlen, "%s", chk.msg);
            errors += chk.errors;
        }
    }
    return errors;
}

}  // namespace

// The q8_1 quantizer through its lane code; chunk: blocks per launch (0: the
// launcher's).  Returns out-of-bounds or misaligned source reads.
extern "C" __attribute__((visibility("default"))) long nq_emu_quantize_q8_1(int in, const void *x, uint64_t nblocks,
                                                                           uint32_t *blocks, uint32_t *status,
                                                                           uint64_t chunk, char *err, int errlen) {
    if (chunk == 0) chunk = nq::Q81_CHUNK;
    switch (in) {
    case 0: return run_q81<0>(x, nblocks, blocks, status, chunk, err, errlen);
    case 1: return run_q81<1>(x, nblocks, blocks, status, chunk, err, errlen);
    case 2: return run_q81<2>(x, nblocks, blocks, status, chunk, err, errlen);
    default: return run_q81<3>(x, nblocks, blocks, status, chunk, err, errlen);
    }
}
#endif  // NQ_EMU_PART
