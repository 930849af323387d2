// k_gemm_kquant.hip -- batched products with q8_1 activations, kquant formats (instantiated per format).
#include "nq_launch.h"

namespace nq {
int launch_gemm_kquant(int fmt, const GvLaunch &L, hipStream_t s) {
    switch (fmt) {
    case Q2_K: return launch_gemm_f<Q2_K>(L, s);
    case Q3_K: return launch_gemm_f<Q3_K>(L, s);
    case Q4_K: return launch_gemm_f<Q4_K>(L, s);
    case Q5_K: return launch_gemm_f<Q5_K>(L, s);
    case Q6_K: return launch_gemm_f<Q6_K>(L, s);
    case Q8_K: return launch_gemm_f<Q8_K>(L, s);
    case IQ4_XS: return launch_gemm_f<IQ4_XS>(L, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
