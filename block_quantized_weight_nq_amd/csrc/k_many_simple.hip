// k_many_simple.hip -- many-tensor decode kernels of the simple family (instantiated per format,
// output type, tile size and store width).
#include "nq_launch.h"

namespace nq {
int launch_many_simple(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s) {
    switch (fmt) {
    case Q4_0: return launch_many_any<Q4_0>(ot, vec, items, n, resident, s);
    case Q4_1: return launch_many_any<Q4_1>(ot, vec, items, n, resident, s);
    case Q5_0: return launch_many_any<Q5_0>(ot, vec, items, n, resident, s);
    case Q5_1: return launch_many_any<Q5_1>(ot, vec, items, n, resident, s);
    case Q8_0: return launch_many_any<Q8_0>(ot, vec, items, n, resident, s);
    case Q8_1: return launch_many_any<Q8_1>(ot, vec, items, n, resident, s);
    case IQ4_NL: return launch_many_any<IQ4_NL>(ot, vec, items, n, resident, s);
    case Q1_0: return launch_many_any<Q1_0>(ot, vec, items, n, resident, s);
    case Q2_0: return launch_many_any<Q2_0>(ot, vec, items, n, resident, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
