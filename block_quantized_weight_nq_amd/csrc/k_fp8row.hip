// k_fp8row.hip -- row-scaled FP8 decode kernels (per scale type and output type).
#include "nq_fp8row.h"

namespace nq {

template <int SK, int OT>
static int launch_f8(const F8Launch &L, hipStream_t stream) {
    const uint64_t total = L.N * L.K;
    constexpr uint64_t OSZ = OT == 0 ? 4 : OT == 3 ? 8 : 2;
    for (uint64_t E0 = 0; E0 < total; E0 += F8_CHUNK) {
        uint32_t grid;
        const F8Args a = f8_chunk_args<OT>(L, E0, &grid);
        // every unit starts at a multiple of 8 values: 16-byte aligned when the
        // launch's output is (for 16-bit outputs; f32/f64 units are 32/64 bytes)
        const bool vec = ((uintptr_t)L.out + E0 * OSZ) % 16 == 0;
        if (vec)
            hipLaunchKernelGGL((k_fp8_row<SK, OT, true>), dim3(grid), dim3(WG), 0, stream, a);
        else
            hipLaunchKernelGGL((k_fp8_row<SK, OT, false>), dim3(grid), dim3(WG), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return 9;  // NQ_ERR_HIP
    }
    return 0;
}

template <int SK>
static int launch_f8_ot(int ot, const F8Launch &L, hipStream_t s) {
    switch (ot) {
    case 0: return launch_f8<SK, 0>(L, s);
    case 1: return launch_f8<SK, 1>(L, s);
    case 2: return launch_f8<SK, 2>(L, s);
    default: return launch_f8<SK, 3>(L, s);
    }
}

int launch_fp8_row(int scale_kind, int ot, const F8Launch &L, hipStream_t s) {
    return scale_kind == 0 ? launch_f8_ot<0>(ot, L, s) : launch_f8_ot<1>(ot, L, s);
}

}  // namespace nq
