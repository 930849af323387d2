// k_many_fp4.hip -- many-tensor decode kernels of the fp4 family (instantiated per format,
// output type, tile size and store width).
#include "nq_launch.h"

namespace nq {
int launch_many_fp4(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s) {
    switch (fmt) {
    case MXFP4: return launch_many_any<MXFP4>(ot, vec, items, n, resident, s);
    case NVFP4_GGUF: return launch_many_any<NVFP4_GGUF>(ot, vec, items, n, resident, s);
    case NVFP4_DIV: return launch_many_any<NVFP4_DIV>(ot, vec, items, n, resident, s);
    default: return 2;  // NQ_ERR_UNKNOWN_FORMAT
    }
}
}  // namespace nq
