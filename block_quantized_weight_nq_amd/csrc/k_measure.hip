// k_measure.hip -- a streaming kernel with a decode's memory traffic and no
// arithmetic: the practical HBM ceiling a decode of the same read and write
// byte counts can reach.
//
// The output is cut into tiles of 256 threads x C 16-byte chunks (C = 1, 2,
// 4 or 8: the output of one 16-bit decode tile of C units per thread), and
// tile t reads its proportional share of the source, chunks
// [t*ns/T, (t+1)*ns/T) of T tiles, with 16-byte loads, each thread taking
// chunks tid, tid + 256, ... of the share (at most C, since the source is no
// larger than the output).  Every thread then stores the XOR of what it
// loaded (one more XOR with the store's index within the thread) to its C
// output chunks, so every load feeds the stores and nothing is optimized
// away.  Loads and stores are non-temporal or ordinary as asked.
#include "nq_launch.h"

namespace nq {

namespace {

template <bool NTL, bool NTS, int C>
__global__ __launch_bounds__(WG) void k_stream(const u32x4 *src, uint64_t nsrc, u32x4 *dst, uint64_t ndst,
                                                uint64_t ntiles) {
    const uint64_t t = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    const uint64_t lo = t * nsrc / ntiles, hi = (t + 1) * nsrc / ntiles;
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (uint32_t k = 0; k < (uint32_t)C; k++) {
        const uint64_t i = lo + (uint64_t)k * WG + tid;
        if (i < hi) {
            if constexpr (NTL)
                acc ^= __builtin_nontemporal_load(src + i);
            else
                acc ^= src[i];
        }
    }
    const uint64_t o0 = t * (uint64_t)(WG * C) + tid;
#pragma unroll
    for (uint32_t k = 0; k < (uint32_t)C; k++) {
        const uint64_t o = o0 + (uint64_t)k * WG;
        if (o < ndst) {
            u32x4 v = acc;
            v.x ^= k;
            if constexpr (NTS)
                __builtin_nontemporal_store(v, dst + o);
            else
                dst[o] = v;
        }
    }
}

template <bool NTL, bool NTS, int C>
int go(const void *src, uint64_t nsrc, void *dst, uint64_t ndst, hipStream_t s) {
    const uint64_t ntiles = (ndst + WG * C - 1) / (WG * C);
    hipLaunchKernelGGL((k_stream<NTL, NTS, C>), dim3((uint32_t)ntiles), dim3(WG), 0, s, (const u32x4 *)src, nsrc,
                       (u32x4 *)dst, ndst, ntiles);
    return hipGetLastError() == hipSuccess ? 0 : 9;  // NQ_ERR_HIP
}

template <bool NTL, bool NTS>
int go_c(int c, const void *src, uint64_t nsrc, void *dst, uint64_t ndst, hipStream_t s) {
    switch (c) {
    case 1: return go<NTL, NTS, 1>(src, nsrc, dst, ndst, s);
    case 2: return go<NTL, NTS, 2>(src, nsrc, dst, ndst, s);
    case 4: return go<NTL, NTS, 4>(src, nsrc, dst, ndst, s);
    default: return go<NTL, NTS, 8>(src, nsrc, dst, ndst, s);
    }
}

}  // namespace

// src_bytes <= dst_bytes, both multiples of 16 and dst_bytes positive, both
// pointers 16-byte aligned, c one of 1, 2, 4, 8, and fewer than 2^31 tiles:
// checked by the caller.
int launch_stream(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes, int c, bool nt_load,
                  bool nt_store, hipStream_t s) {
    const uint64_t nsrc = src_bytes / 16, ndst = dst_bytes / 16;
    if (nt_load)
        return nt_store ? go_c<true, true>(c, src, nsrc, dst, ndst, s) : go_c<true, false>(c, src, nsrc, dst, ndst, s);
    return nt_store ? go_c<false, true>(c, src, nsrc, dst, ndst, s) : go_c<false, false>(c, src, nsrc, dst, ndst, s);
}

}  // namespace nq
