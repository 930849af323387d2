// k_simple.hip -- decode kernels of the simple family (instantiated per format and output type).
#include "nq_launch.h"

namespace nq {
int launch_simple(int fmt, int ot, const LaunchArgs &L, hipStream_t s) {
    switch (fmt) {
    case Q4_0: return launch_any<Q4_0>(ot, L, s);
    case Q4_1: return launch_any<Q4_1>(ot, L, s);
    case Q5_0: return launch_any<Q5_0>(ot, L, s);
    case Q5_1: return launch_any<Q5_1>(ot, L, s);
    case Q8_0: return launch_any<Q8_0>(ot, L, s);
    case Q8_1: return launch_any<Q8_1>(ot, L, s);
    case IQ4_NL: return launch_any<IQ4_NL>(ot, L, s);
    case Q1_0: return launch_any<Q1_0>(ot, L, s);
    case Q2_0: return launch_any<Q2_0>(ot, L, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
