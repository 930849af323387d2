// k_ternary.hip -- decode kernels of the ternary family (instantiated per format and output type).
#include "nq_launch.h"

namespace nq {
int launch_ternary(int fmt, int ot, const LaunchArgs &L, hipStream_t s) {
    switch (fmt) {
    case TQ1_0: return launch_any<TQ1_0>(ot, L, s);
    case TQ2_0: return launch_any<TQ2_0>(ot, L, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
