// nq_launch.h -- internal: per-family launch entry points.
#pragma once
#include <hip/hip_runtime.h>
#include "nq_kernel.h"

namespace nq {
int launch_simple(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_kquant(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_iq(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_fp4(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_ternary(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
}  // namespace nq
