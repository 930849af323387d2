// k_gqenc.hip -- grouped_absmax encoder kernels (per scheme and source type).
#include "nq_gqenc.h"

namespace nq {

// Clears the status word, ordered on the stream (a kernel rather than a
// memset node, so that a captured graph replays it reliably).
__global__ void k_gq_clear_status(uint32_t *status) { *status = 0u; }

template <int S, int IN>
static int launch_gq(const GqLaunch &L, hipStream_t stream) {
    constexpr uint64_t ESZ = IN == 0 ? 4 : IN == 3 ? 8 : 2;
    hipLaunchKernelGGL(k_gq_clear_status, dim3(1), dim3(1), 0, stream, L.status);
    if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
    // 16-byte source loads need every lane's 8 values on a 16-byte boundary;
    // 8-byte code stores need every row on a 4-byte boundary
    const bool vin = (uintptr_t)L.x % 16 == 0 && (L.K * ESZ) % 16 == 0;
    const bool vout = (uintptr_t)L.codes % 4 == 0 && L.K % 4 == 0;
    for (uint64_t r0 = 0; r0 < L.N;) {
        uint64_t rows;
        uint32_t grid;
        const GqArgs a = gq_chunk_args<S, IN>(L, r0, &rows, &grid);
        if (vin && vout)
            hipLaunchKernelGGL((k_grouped_absmax<S, IN, true, true>), dim3(grid), dim3(WG), 0, stream, a);
        else if (vin)
            hipLaunchKernelGGL((k_grouped_absmax<S, IN, true, false>), dim3(grid), dim3(WG), 0, stream, a);
        else if (vout)
            hipLaunchKernelGGL((k_grouped_absmax<S, IN, false, true>), dim3(grid), dim3(WG), 0, stream, a);
        else
            hipLaunchKernelGGL((k_grouped_absmax<S, IN, false, false>), dim3(grid), dim3(WG), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
        r0 += rows;
    }
    return 0;
}

template <int S>
static int launch_gq_in(int in_dtype, const GqLaunch &L, hipStream_t s) {
    switch (in_dtype) {
    case 0: return launch_gq<S, 0>(L, s);
    case 1: return launch_gq<S, 1>(L, s);
    case 2: return launch_gq<S, 2>(L, s);
    default: return launch_gq<S, 3>(L, s);
    }
}

int launch_grouped_absmax(int scheme, int in_dtype, const GqLaunch &L, hipStream_t s) {
    switch (scheme) {
    case 0: return launch_gq_in<0>(in_dtype, L, s);
    case 1: return launch_gq_in<1>(in_dtype, L, s);
    case 2: return launch_gq_in<2>(in_dtype, L, s);
    default: return launch_gq_in<3>(in_dtype, L, s);
    }
}

}  // namespace nq
