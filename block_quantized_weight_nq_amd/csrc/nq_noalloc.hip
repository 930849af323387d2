// nq_noalloc.hip -- the batched product without a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The workspace nq_gemm_q8_1 takes from its caller (K-split partial outputs,
// the once-per-call weight rewrite) lives here in a file-scope device array
// of NQ_GEMM_SCRATCH_BYTES.  The HIP runtime gives every GPU the library's
// code is loaded on its own copy of the array, reserved at load and held
// until the process ends; its device address on each GPU comes from
// hipGetSymbolAddress, called once per device with that device current.  In
// host code the array's name is only a host-side stand-in: kernels get the
// per-device address, never the name.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/nq.h"

#define NQ_API extern "C" __attribute__((visibility("default")))

namespace {

static __device__ __align__(256) uint8_t scratch[NQ_GEMM_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> g_scratch[MAX_DEVICES];
std::mutex g_scratch_lock;

// The scratch array's device address on the current device (looked up on
// the device's first call), or NULL if the runtime cannot give it.
void *device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> hold(g_scratch_lock);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        g_scratch[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace

NQ_API int nq_gemm_q8_1_noalloc(int32_t format, const void *weight, uint64_t nbytes, int64_t N, int64_t K,
                                const void *xq, int64_t M, float *y, hipStream_t stream) {
    const int st = nq_validate_gemm_q8_1(format, nbytes, N, K, M);
    if (st != NQ_OK) return st;
    if (!weight || !xq || !y) return NQ_ERR_NULL_ARG;
    if ((uintptr_t)xq % 4 != 0 || (uintptr_t)y % 4 != 0) return NQ_ERR_MISALIGNED;
    uint64_t need = 0;
    const int sw = nq_gemm_q8_1_workspace(format, N, K, M, &need);
    if (sw != NQ_OK) return sw;
    if (need > (uint64_t)NQ_GEMM_SCRATCH_BYTES) return NQ_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        ws = device_scratch();
        if (!ws) return NQ_ERR_HIP;
    }
    return nq_gemm_q8_1(format, weight, nbytes, N, K, xq, M, y, ws, need, stream);
}
