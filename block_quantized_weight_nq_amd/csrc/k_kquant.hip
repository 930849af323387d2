// k_kquant.hip -- decode kernels of the kquant family (instantiated per format and output type).
#include "nq_launch.h"

namespace nq {
int launch_kquant(int fmt, int ot, const LaunchArgs &L, hipStream_t s) {
    switch (fmt) {
    case Q2_K: return launch_any<Q2_K>(ot, L, s);
    case Q3_K: return launch_any<Q3_K>(ot, L, s);
    case Q4_K: return launch_any<Q4_K>(ot, L, s);
    case Q5_K: return launch_any<Q5_K>(ot, L, s);
    case Q6_K: return launch_any<Q6_K>(ot, L, s);
    case Q8_K: return launch_any<Q8_K>(ot, L, s);
    case IQ4_XS: return launch_any<IQ4_XS>(ot, L, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
