// k_q8_1.hip -- q8_1 activation quantizer kernels (per source type).
#include "nq_launch.h"

namespace nq {

// Clears the status word, ordered on the stream (a kernel rather than a
// memset node, so that a captured graph replays it reliably).
__global__ void k_q81_clear_status(uint32_t *status) { *status = 0u; }

template <int IN>
static int launch_q81(const Q81Launch &L, hipStream_t stream) {
    constexpr uint64_t ESZ = IN == 0 ? 4 : IN == 3 ? 8 : 2;
    constexpr uint64_t LPB = 32 / gq_vpl<IN>();
    hipLaunchKernelGGL(k_q81_clear_status, dim3(1), dim3(1), 0, stream, L.status);
    if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
    // 16-byte source loads need the source on a 16-byte boundary (each lane's
    // 32 bytes then are)
    const bool vin = (uintptr_t)L.x % 16 == 0;
    for (uint64_t b0 = 0; b0 < L.nblocks; b0 += Q81_CHUNK) {
        Q81Args a;
        a.x = (const uint8_t *)L.x + b0 * 32 * ESZ;
        a.blocks = L.blocks + b0 * 9;
        a.status = L.status;
        a.nblocks = (uint32_t)(L.nblocks - b0 < Q81_CHUNK ? L.nblocks - b0 : Q81_CHUNK);
        const uint32_t grid = (uint32_t)((a.nblocks * LPB + WG - 1) / WG);
        if (vin)
            hipLaunchKernelGGL((k_quantize_q8_1<IN, true>), dim3(grid), dim3(WG), 0, stream, a);
        else
            hipLaunchKernelGGL((k_quantize_q8_1<IN, false>), dim3(grid), dim3(WG), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
    }
    return 0;
}

int launch_quantize_q8_1(int in_dtype, const Q81Launch &L, hipStream_t s) {
    switch (in_dtype) {
    case 0: return launch_q81<0>(L, s);
    case 1: return launch_q81<1>(L, s);
    case 2: return launch_q81<2>(L, s);
    default: return launch_q81<3>(L, s);
    }
}

}  // namespace nq
