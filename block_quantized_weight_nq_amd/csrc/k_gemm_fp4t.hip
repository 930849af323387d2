// k_gemm_fp4t.hip -- batched products with q8_1 activations, FP4 and ternary formats (instantiated per format).
#include "nq_launch.h"

namespace nq {
int launch_gemm_fp4t(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s) {
    switch (fmt) {
    case MXFP4: return launch_gemm_f<MXFP4>(L, ws, ws_bytes, s);
    case NVFP4_GGUF: return launch_gemm_f<NVFP4_GGUF>(L, ws, ws_bytes, s);
    case TQ1_0: return launch_gemm_f<TQ1_0>(L, ws, ws_bytes, s);
    case TQ2_0: return launch_gemm_f<TQ2_0>(L, ws, ws_bytes, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
