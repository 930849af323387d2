// k_fp4.hip -- decode kernels of the fp4 family (instantiated per format and output type).
#include "nq_launch.h"

namespace nq {
int launch_fp4(int fmt, int ot, const LaunchArgs &L, hipStream_t s) {
    switch (fmt) {
    case MXFP4: return launch_any<MXFP4>(ot, L, s);
    case NVFP4_GGUF: return launch_any<NVFP4_GGUF>(ot, L, s);
    case NVFP4_DIV: return launch_any<NVFP4_DIV>(ot, L, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
