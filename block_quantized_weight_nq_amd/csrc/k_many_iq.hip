// k_many_iq.hip -- many-tensor decode kernels of the iq family (instantiated per format,
// output type, tile size and store width).
#include "nq_launch.h"

namespace nq {
int launch_many_iq(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s) {
    switch (fmt) {
    case IQ2_XXS: return launch_many_any<IQ2_XXS>(ot, vec, items, n, resident, s);
    case IQ2_XS: return launch_many_any<IQ2_XS>(ot, vec, items, n, resident, s);
    case IQ2_S: return launch_many_any<IQ2_S>(ot, vec, items, n, resident, s);
    case IQ3_XXS: return launch_many_any<IQ3_XXS>(ot, vec, items, n, resident, s);
    case IQ3_S: return launch_many_any<IQ3_S>(ot, vec, items, n, resident, s);
    case IQ1_S: return launch_many_any<IQ1_S>(ot, vec, items, n, resident, s);
    case IQ1_M: return launch_many_any<IQ1_M>(ot, vec, items, n, resident, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
