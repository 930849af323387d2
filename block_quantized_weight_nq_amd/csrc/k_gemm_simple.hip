// k_gemm_simple.hip -- batched products with q8_1 activations, simple formats (instantiated per format).
#include "nq_launch.h"

namespace nq {
int launch_gemm_simple(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s) {
    switch (fmt) {
    case Q4_0: return launch_gemm_f<Q4_0>(L, ws, ws_bytes, s);
    case Q4_1: return launch_gemm_f<Q4_1>(L, ws, ws_bytes, s);
    case Q5_0: return launch_gemm_f<Q5_0>(L, ws, ws_bytes, s);
    case Q5_1: return launch_gemm_f<Q5_1>(L, ws, ws_bytes, s);
    case Q8_0: return launch_gemm_f<Q8_0>(L, ws, ws_bytes, s);
    case Q8_1: return launch_gemm_f<Q8_1>(L, ws, ws_bytes, s);
    case IQ4_NL: return launch_gemm_f<IQ4_NL>(L, ws, ws_bytes, s);
    case Q1_0: return launch_gemm_f<Q1_0>(L, ws, ws_bytes, s);
    case Q2_0: return launch_gemm_f<Q2_0>(L, ws, ws_bytes, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
