// k_iq.hip -- decode kernels of the iq family (instantiated per format and output type).
#include "nq_launch.h"

namespace nq {
int launch_iq(int fmt, int ot, const LaunchArgs &L, hipStream_t s) {
    switch (fmt) {
    case IQ2_XXS: return launch_any<IQ2_XXS>(ot, L, s);
    case IQ2_XS: return launch_any<IQ2_XS>(ot, L, s);
    case IQ2_S: return launch_any<IQ2_S>(ot, L, s);
    case IQ3_XXS: return launch_any<IQ3_XXS>(ot, L, s);
    case IQ3_S: return launch_any<IQ3_S>(ot, L, s);
    case IQ1_S: return launch_any<IQ1_S>(ot, L, s);
    case IQ1_M: return launch_any<IQ1_M>(ot, L, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
