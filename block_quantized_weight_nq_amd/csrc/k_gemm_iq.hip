// k_gemm_iq.hip -- batched products with q8_1 activations, iq formats (instantiated per format).
#include "nq_launch.h"

namespace nq {
int launch_gemm_iq(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s) {
    switch (fmt) {
    case IQ2_XXS: return launch_gemm_f<IQ2_XXS>(L, ws, ws_bytes, s);
    case IQ2_XS: return launch_gemm_f<IQ2_XS>(L, ws, ws_bytes, s);
    case IQ2_S: return launch_gemm_f<IQ2_S>(L, ws, ws_bytes, s);
    case IQ3_XXS: return launch_gemm_f<IQ3_XXS>(L, ws, ws_bytes, s);
    case IQ3_S: return launch_gemm_f<IQ3_S>(L, ws, ws_bytes, s);
    case IQ1_S: return launch_gemm_f<IQ1_S>(L, ws, ws_bytes, s);
    case IQ1_M: return launch_gemm_f<IQ1_M>(L, ws, ws_bytes, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
