// k_many_ternary.hip -- many-tensor decode kernels of the ternary family (instantiated per format,
// output type, tile size and store width).
#include "nq_launch.h"

namespace nq {
int launch_many_ternary(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s) {
    switch (fmt) {
    case TQ1_0: return launch_many_any<TQ1_0>(ot, vec, items, n, resident, s);
    case TQ2_0: return launch_many_any<TQ2_0>(ot, vec, items, n, resident, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
