// k_gemm_kquant.hip -- batched products with q8_1 activations, kquant formats (instantiated per format).
#include "nq_launch.h"

namespace nq {
int launch_gemm_kquant(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s) {
    switch (fmt) {
    case Q2_K: return launch_gemm_f<Q2_K>(L, ws, ws_bytes, s);
    case Q3_K: return launch_gemm_f<Q3_K>(L, ws, ws_bytes, s);
    case Q4_K: return launch_gemm_f<Q4_K>(L, ws, ws_bytes, s);
    case Q5_K: return launch_gemm_f<Q5_K>(L, ws, ws_bytes, s);
    case Q6_K: return launch_gemm_f<Q6_K>(L, ws, ws_bytes, s);
    case Q8_K: return launch_gemm_f<Q8_K>(L, ws, ws_bytes, s);
    case IQ4_XS: return launch_gemm_f<IQ4_XS>(L, ws, ws_bytes, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
