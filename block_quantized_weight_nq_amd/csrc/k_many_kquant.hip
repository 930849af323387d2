// k_many_kquant.hip -- many-tensor decode kernels of the kquant family (instantiated per format,
// output type, tile size and store width).
#include "nq_launch.h"

namespace nq {
int launch_many_kquant(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s) {
    switch (fmt) {
    case Q2_K: return launch_many_any<Q2_K>(ot, vec, items, n, resident, s);
    case Q3_K: return launch_many_any<Q3_K>(ot, vec, items, n, resident, s);
    case Q4_K: return launch_many_any<Q4_K>(ot, vec, items, n, resident, s);
    case Q5_K: return launch_many_any<Q5_K>(ot, vec, items, n, resident, s);
    case Q6_K: return launch_many_any<Q6_K>(ot, vec, items, n, resident, s);
    case Q8_K: return launch_many_any<Q8_K>(ot, vec, items, n, resident, s);
    case IQ4_XS: return launch_many_any<IQ4_XS>(ot, vec, items, n, resident, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
