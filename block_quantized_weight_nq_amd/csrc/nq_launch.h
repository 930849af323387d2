// nq_launch.h -- internal: per-family launch entry points.
#pragma once
#include <hip/hip_runtime.h>
#include "nq_gemm.h"
#include "nq_kernel.h"

namespace nq {
int launch_simple(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_kquant(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_iq(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_fp4(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_ternary(int fmt, int ot, const LaunchArgs &L, hipStream_t s);
int launch_gemv_simple(int fmt, const GvLaunch &L, hipStream_t s);
int launch_gemv_kquant(int fmt, const GvLaunch &L, hipStream_t s);
int launch_gemv_iq(int fmt, const GvLaunch &L, hipStream_t s);
int launch_gemv_fp4t(int fmt, const GvLaunch &L, hipStream_t s);
int launch_gemm_simple(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s);
int launch_gemm_kquant(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s);
int launch_gemm_iq(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s);
int launch_gemm_fp4t(int fmt, const GvLaunch &L, void *ws, uint64_t ws_bytes, hipStream_t s);
int launch_quantize_q8_1(int in_dtype, const Q81Launch &L, hipStream_t s);
int launch_many_simple(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s);
int launch_many_kquant(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s);
int launch_many_iq(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s);
int launch_many_fp4(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s);
int launch_many_ternary(int fmt, int ot, bool vec, const ManyItem *items, int n, uint32_t resident, hipStream_t s);
int launch_stream(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes, int c, bool nt_load,
                  bool nt_store, hipStream_t s);
}  // namespace nq
