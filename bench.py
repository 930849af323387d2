#!/usr/bin/env python3
"""Decode throughput of packed block-quantized weights on one MI355X.

A step decodes the whole Llama-3-8B-shaped weight set (226 tensors; formats
q4_k, q6_k, q8_0, nvfp4, tq2_0 in rotation) to bf16 on one stream, with every
payload already resident in HBM: one nq_dequantize_packed_many call, which
decodes the tensors of each format in one launch.  The same step made of 226
single-tensor calls (nq_dequantize_packed) is timed beside it.  The JSON line
reports:

  value          (payload + output bytes of the step) / (seconds per step)
  roofline       the dominant kernel (most total time) against MI355X HBM
                 peak: its algorithmic bytes per launch over its mean launch
                 duration, timed with HIP events on the launch stream; beside
                 it the measured ceiling of a plain streaming kernel with the
                 same read and write bytes (nq_measure_stream)
  cpu_baseline   the oracle, single-threaded and pinned to one host core, on
                 a bounded sample (the first third of each tensor's blocks)
  per_format     every format of the step; every one of the 28 formats at
                 [14336, 4096] -> bf16; the remaining workloads (q8_0/q4_0
                 [64, 4096] -> f32, launch-bound; q4_k/q6_k [4096, 4096];
                 mxfp4/nvfp4 [14336, 4096]; the IQ set [4096, 14336] to f32
                 and bf16), each timed over rotating replicas so no launch
                 reads a payload out of a warm cache

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --formats gguf:q6_k,nvfp4 --shapes 14336x4096,4096x4096   (profiling target)
"""
import argparse
import json
import math
import os
import sys
import time

METRIC = "decode GB/s (payload+output) per format & % of HBM peak, 1×MI355X"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
OUT_CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
OUT_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8}


# The sources the decode kernels are built from (the kernels the counter profile covers).
DECODE_SOURCES = ["iq_grids.h", "nq_decode.h", "nq_kernel.h", "k_simple.hip", "k_kquant.hip", "k_iq.hip",
                  "k_fp4.hip", "k_ternary.hip", "k_many_simple.hip", "k_many_kquant.hip", "k_many_iq.hip",
                  "k_many_fp4.hip", "k_many_ternary.hip"]


def sources_sha256():
    """Hash of the decode kernels' sources without comments (the build the counter profile was taken on)."""
    import re
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "block_quantized_weight_nq_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in DECODE_SOURCES)
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        # comments and blank lines do not change the kernels
        code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()


def profiled_traffic(kernel_fmt):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE profile (copy-calibrated),
    or None when that profile was taken on other kernel sources."""
    import glob
    here = os.path.dirname(os.path.abspath(__file__))
    for path in sorted(glob.glob(os.path.join(here, "profiles", "traffic_*.md"))):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line.startswith("TRAFFIC "):
                    rec = json.loads(line[len("TRAFFIC "):])
                    if rec.get("sources_sha256") == sources_sha256() and kernel_fmt in rec.get("kernels", {}):
                        return rec["kernels"][kernel_fmt]["traffic_bytes"]
    return None


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


class Tensor:
    """One resident payload and its output buffer."""

    def __init__(self, name, fmt, shape, recipe, seed, dtype, staging, torch, nq, synth, divisors=1):
        info = nq.format_query(fmt)
        self.name, self.fmt, self.shape, self.dtype = name, fmt, list(shape), dtype
        self.fid = info.id
        nel = 1
        for d in shape:
            nel *= d
        self.nelems = nel
        self.nblocks = nel // info.block_values
        self.divisors = divisors if info.trailer_bytes else 0
        self.nbytes = self.nblocks * info.block_bytes + 4 * self.divisors
        host = staging[: self.nbytes]
        if self.nblocks:
            synth.fill_into(fmt, self.nblocks, seed, recipe, host.data_ptr())
        for j in range(self.divisors):  # one binary32 divisor per stacked source
            bits = synth.divisor_bits(seed + j)
            o = self.nblocks * info.block_bytes + 4 * j
            host[o:o + 4] = torch.tensor([(bits >> (8 * i)) & 0xFF for i in range(4)], dtype=torch.uint8)
        self.payload = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda:0")
        self.payload.copy_(host, non_blocking=False)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}[dtype]
        self.out = torch.empty(nel, dtype=tdt, device="cuda:0")
        self.algo_bytes = self.nbytes + nel * OUT_SIZE[dtype]
        self.seed, self.recipe = seed, recipe

    def desc(self):
        return (self.fid, self.payload.data_ptr(), self.nbytes, self.shape, self.out.data_ptr())

    def launch(self, nq, stream_handle):
        if self.divisors > 1:
            st = nq.dequantize_nvfp4_stacked_raw(self.payload.data_ptr(), self.nbytes, self.shape, self.divisors,
                                                 OUT_CODES[self.dtype], self.out.data_ptr(), stream_handle)
        else:
            st = nq.dequantize_packed_raw(self.fid, self.payload.data_ptr(), self.nbytes, self.shape,
                                          OUT_CODES[self.dtype], self.out.data_ptr(), stream_handle)
        if st != 0:
            raise nq.NqError(st, self.name)


def staging_buffer(torch, tensors, nq):
    need = 0
    for _, fmt, shape, _, _ in tensors:
        info = nq.format_query(fmt)
        nel = math.prod(shape)
        need = max(need, nel // info.block_values * info.block_bytes + info.trailer_bytes)
    return torch.empty(need, dtype=torch.uint8, pin_memory=True)


def capture(torch, nq, items):
    """A HIP graph holding one launch per item, in order, on torch's capture stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for it in items:
            it.launch(nq, h)
    return g


def time_graph(torch, g, reps, warmup=1):
    """Mean milliseconds per replay, timed with events on the replay stream."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(reps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / reps
    return start.elapsed_time(end) / reps, wall


def time_eager(torch, nq, items, steps, warmup):
    """Wall and event milliseconds per pass of eager launches (no per-launch events)."""
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    for _ in range(warmup):
        for it in items:
            it.launch(nq, handle)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        for it in items:
            it.launch(nq, handle)
    end.record(stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, start.elapsed_time(end) / steps


def capture_many(torch, call):
    """A HIP graph holding one many-tensor call on torch's capture stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.run(torch.cuda.current_stream().cuda_stream)
    return g


def time_eager_many(torch, call, steps, warmup):
    """Wall and event milliseconds per eager many-tensor call."""
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    for _ in range(warmup):
        call.run(handle)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        call.run(handle)
    end.record(stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, start.elapsed_time(end) / steps


def many_launches(n):
    """Launches of a many-tensor call over n tensors of one format (64 to a launch)."""
    return (n + 63) // 64


def per_format_times(torch, nq, items, reps):
    """Per format: one many-tensor call over the step's tensors of that format
    (one launch per 64 tensors), graph-captured and timed by events on the
    replay stream."""
    out = {}
    for fmt in dict.fromkeys(it.fmt for it in items):
        sel = [it for it in items if it.fmt == fmt]
        call = nq.ManyCall([it.desc() for it in sel], OUT_CODES["bf16"])
        g = capture_many(torch, call)
        ms, _ = time_graph(torch, g, reps)
        nbytes = sum(it.algo_bytes for it in sel)
        nl = many_launches(len(sel))
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[fmt] = {"gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "tensors": len(sel),
                    "launches": nl, "mean_launch_us": round(ms * 1e3 / nl, 3), "bytes_per_launch": round(nbytes / nl),
                    "read_bytes_per_launch": round(sum(it.nbytes for it in sel) / nl), "total_ms": ms}
        del g
    return out


STREAM_CONFIGS = [(c, f) for c in (1, 2, 4, 8) for f in (3, 2)]  # chunks per thread; NT load (1) and NT store (2)


def stream_ceiling(torch, nq, read_bytes, write_bytes, launches=40, configs=STREAM_CONFIGS):
    """nq_measure_stream (the decode's traffic, no arithmetic) over a cold
    rotation, in each tile size and cache policy of `configs`: the best GB/s
    of read + write bytes per mean launch time, with every configuration's."""
    rb, wb = -(-read_bytes // 16) * 16, -(-write_bytes // 16) * 16
    reps = cold_replicas(rb, rb + wb) if rb + wb < (2 << 30) else 1
    launches = max(launches, reps)
    bufs = [(torch.empty(rb, dtype=torch.uint8, device="cuda:0").fill_(r + 1),
             torch.empty(wb, dtype=torch.uint8, device="cuda:0")) for r in range(reps)]
    runs = {}
    for c, flags in configs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h = torch.cuda.current_stream().cuda_stream
            for i in range(launches):
                src, dst = bufs[i % reps]
                st = nq.measure_stream_raw(src.data_ptr(), rb, dst.data_ptr(), wb, c, flags, h)
                if st != 0:
                    raise nq.NqError(st, "measure_stream")
        ms, _ = time_graph(torch, g, 3)
        del g
        mean_ms = ms / launches
        runs[f"c{c}{'_ntl' if flags & 1 else ''}{'_nts' if flags & 2 else ''}"] = \
            (round((rb + wb) / (mean_ms * 1e-3) / 1e9, 1), round(mean_ms * 1e3, 3))
    del bufs
    torch.cuda.empty_cache()
    best = max(runs, key=lambda k: runs[k][0])
    return {"gbps": runs[best][0], "frac_hbm_peak": round(runs[best][0] / HBM_PEAK_GBPS, 4), "read_bytes": rb,
            "write_bytes": wb, "mean_launch_us": runs[best][1], "replicas": reps, "best": best,
            "kernel": "k_stream (nq_measure_stream)", "gbps_by_config": {k: v[0] for k, v in runs.items()}}


def cold_replicas(read_bytes, total_bytes, cap=2048):
    """Replicas for a rotation that reads HBM on every launch: the read
    buffers alone pass 1 GiB (four times MI355X's 256 MB last-level cache,
    which keeps payloads that ordinary loads bring in) and all buffers pass
    2 GiB."""
    return max(2, min(cap, max(math.ceil((1 << 30) / max(1, read_bytes)), math.ceil((2 << 30) / total_bytes))))


def rotating_measurement(torch, nq, synth, name, fmt, shape, recipe, seed, dtype, staging, launches=60,
                         divisors=1):
    """Mean launch time of one workload over a cold rotation of replicas
    (cold_replicas; at least one launch per replica)."""
    first = Tensor(name, fmt, shape, recipe, seed, dtype, staging, torch, nq, synth, divisors)
    reps = cold_replicas(first.nbytes, first.algo_bytes)
    launches = max(launches, reps)
    items = [first]
    for r in range(1, reps):  # same payload bytes, own buffers
        t = Tensor.__new__(Tensor)
        t.__dict__.update(first.__dict__)
        t.payload = first.payload.clone()
        t.out = torch.empty_like(first.out)
        items.append(t)
    order = [items[i % reps] for i in range(launches)]
    g = capture(torch, nq, order)
    ms, _ = time_graph(torch, g, 3)
    mean_ms = ms / launches
    gbps = first.algo_bytes / (mean_ms * 1e-3) / 1e9
    res = {"shape": shape, "out": dtype, "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "mean_launch_us": round(mean_ms * 1e3, 3), "replicas": reps,
           "elements_per_s": round(first.nelems / (mean_ms * 1e-3), 1), "bytes_per_launch": first.algo_bytes}
    del g, items, order, first
    torch.cuda.empty_cache()
    return res


def fp8_row_measurement(torch, nq, fmt, shape, dtype, launches=60, seed=0x6E7F8000):
    """Row-scaled FP8 decode over rotating replicas: random code words with the
    NaN words replaced, positive normal scale words ([2^-9, 2^-5) for bfloat16,
    [2^-8, 2^-4) for binary16)."""
    import numpy as np
    N, K = shape
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=N * K, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 0x01
    lo, hi = (0x3B00, 0x3D00) if fmt.endswith("bf16") else (0x1C00, 0x2C00)
    scales = rng.integers(lo, hi, size=N).astype("<u2")
    host = torch.from_numpy(np.concatenate([codes, scales.view(np.uint8)]))
    nbytes = host.numel()
    out_bytes = N * K * OUT_SIZE[dtype]
    reps = cold_replicas(nbytes, nbytes + out_bytes)
    launches = max(launches, reps)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}[dtype]
    items = [(host.to("cuda:0"), torch.empty(N * K, dtype=tdt, device="cuda:0")) for _ in range(reps)]
    kind = nq.FP8_ROW_KINDS[fmt]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(launches):
            p, o = items[i % reps]
            st = nq.dequantize_fp8_row_raw(kind, p.data_ptr(), nbytes, shape, OUT_CODES[dtype], o.data_ptr(), h)
            if st != 0:
                raise nq.NqError(st, fmt)
    ms, _ = time_graph(torch, g, 3)
    mean_ms = ms / launches
    gbps = (nbytes + out_bytes) / (mean_ms * 1e-3) / 1e9
    res = {"shape": shape, "out": dtype, "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "mean_launch_us": round(mean_ms * 1e3, 3), "replicas": reps,
           "elements_per_s": round(N * K / (mean_ms * 1e-3), 1), "bytes_per_launch": nbytes + out_bytes}
    del g, items
    torch.cuda.empty_cache()
    return res


def gq_measurement(torch, nq, scheme, shape, in_dtype, launches=60, seed=0x6E7A6000):
    """grouped_absmax encoder over rotating replicas of a normal source with
    row magnitudes 2^-8 .. 2^4; bytes = source + codes + binary16 scales."""
    import numpy as np
    N, K = shape
    sid, G = nq.GQ_SCHEMES[scheme]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}[in_dtype]
    rng = np.random.default_rng(seed)
    x = torch.from_numpy((rng.standard_normal((N, K)) * np.exp2(rng.integers(-8, 4, (N, 1)))).astype(np.float32))
    x = x.to(tdt)
    ng = (K + G - 1) // G
    nbytes = x.numel() * x.element_size() + N * K + 2 * N * ng
    reps = cold_replicas(x.numel() * x.element_size(), nbytes)
    launches = max(launches, reps)
    items = [(x.to("cuda:0"), torch.empty((N, K), dtype=torch.int8, device="cuda:0"),
              torch.empty((N, ng), dtype=torch.int16, device="cuda:0"),
              torch.empty(1, dtype=torch.int32, device="cuda:0")) for _ in range(reps)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(launches):
            xs, c, sc, st = items[i % reps]
            rc = nq.quantize_grouped_absmax_raw(sid, xs.data_ptr(), shape, nq.DTYPE_CODES[in_dtype], c.data_ptr(),
                                                sc.data_ptr(), st.data_ptr(), h)
            if rc != 0:
                raise nq.NqError(rc, scheme)
    ms, _ = time_graph(torch, g, 3)
    torch.cuda.synchronize()
    if any(int(it[3].item()) for it in items):
        raise RuntimeError("grouped_absmax reported a failure on the benchmark source")
    mean_ms = ms / launches
    gbps = nbytes / (mean_ms * 1e-3) / 1e9
    res = {"shape": shape, "in": in_dtype, "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "mean_launch_us": round(mean_ms * 1e3, 3), "replicas": reps,
           "elements_per_s": round(N * K / (mean_ms * 1e-3), 1), "bytes_per_launch": nbytes,
           "note": "two launches per call (status clear + encoder)"}
    del g, items
    torch.cuda.empty_cache()
    return res


def gemv_measurement(torch, nq, synth, fmt, shape, M, launches=60, seed=0x6E7C7000):
    """Products with q8_1 activations (nq_gemv_q8_1) over rotating replicas of
    a weight [N, K]; bytes = weight payload + q8_1 activation blocks + binary32
    output, each counted once per launch (the activation is read from cache by
    every workgroup)."""
    import numpy as np
    N, K = shape
    info = nq.format_query(fmt)
    nbytes_w = N * K // info.block_values * info.block_bytes
    host = synth.payload(fmt, N * K // info.block_values, seed, synth.binade(-6, -2, False))
    w0 = torch.from_numpy(host).to("cuda:0")
    reps = cold_replicas(nbytes_w, nbytes_w)
    launches = max(launches, reps)
    ws = [w0] + [w0.clone() for _ in range(reps - 1)]
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to("cuda:0")
    xq, _ = nq.quantize_q8_1(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(launches):
            rc = nq.gemv_q8_1_raw(info.id, ws[i % reps].data_ptr(), nbytes_w, N, K, xq.data_ptr(), M, y.data_ptr(), h)
            if rc != 0:
                raise nq.NqError(rc, fmt)
    ms, _ = time_graph(torch, g, 3)
    mean_ms = ms / launches
    nbytes = nbytes_w + xq.numel() + 4 * M * N
    gbps = nbytes / (mean_ms * 1e-3) / 1e9
    res = {"shape": shape, "M": M, "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
           "weight_gbps": round(nbytes_w / (mean_ms * 1e-3) / 1e9, 1), "mean_launch_us": round(mean_ms * 1e3, 3),
           "replicas": reps, "weights_per_s": round(N * K / (mean_ms * 1e-3), 1), "bytes_per_launch": nbytes}
    del g, ws, w0
    torch.cuda.empty_cache()
    return res


GEMV_CASES = [("gguf:q4_k", 1), ("gguf:q6_k", 1), ("gguf:q8_0", 1), ("gguf:q4_0", 1), ("gguf:iq4_xs", 1),
              ("gguf:mxfp4", 1), ("gguf:iq2_xxs", 1), ("gguf:tq2_0", 1), ("gguf:q4_k", 8), ("gguf:q8_0", 8)]


# Batched products (nq_gemm_q8_1, more than 8 activation rows): integer
# operations 2 * M * N * K per launch.  The 8-bit matrix cores' dense peak is
# 5.0 POP/s; the binding limit is the vector ALU, which scales every exact
# 32-value dot product in binary32 (convert, product of the two scales,
# fused multiply-add: 3 wave instructions per output and span).  256 CUs x 4
# SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane operations/s, / 3 per 32
# multiply-adds, x 2 operations each = 838.9 TOP/s.
MFMA_I8_PEAK_TOPS = 5000.0
GEMM_ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 3 * 32 * 2 / 1e12


def gemm_measurement(torch, nq, synth, fmt, shape, M, launches=20, seed=0x6E7C8000):
    """Batched products with q8_1 activations over rotating weight replicas;
    TOP/s = 2 M N K per mean launch time."""
    import numpy as np
    N, K = shape
    info = nq.format_query(fmt)
    nbytes_w = N * K // info.block_values * info.block_bytes
    host = synth.payload(fmt, N * K // info.block_values, seed, synth.binade(-6, -2, False))
    w0 = torch.from_numpy(host).to("cuda:0")
    reps = cold_replicas(nbytes_w, nbytes_w)
    launches = max(launches, reps)
    ws = [w0] + [w0.clone() for _ in range(reps - 1)]
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to("cuda:0")
    xq, _ = nq.quantize_q8_1(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    st, ws_bytes = nq.gemm_q8_1_workspace(info.id, N, K, M)
    if st != 0:
        raise nq.NqError(st, fmt)
    work = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(launches):
            rc = nq.gemm_q8_1_raw(info.id, ws[i % reps].data_ptr(), nbytes_w, N, K, xq.data_ptr(), M, y.data_ptr(),
                                  work.data_ptr(), ws_bytes, h)
            if rc != 0:
                raise nq.NqError(rc, fmt)
    ms, _ = time_graph(torch, g, 3)
    mean_ms = ms / launches
    tops = 2.0 * M * N * K / (mean_ms * 1e-3) / 1e12
    res = {"shape": shape, "M": M, "tops": round(tops, 1), "frac_alu_peak": round(tops / GEMM_ALU_PEAK_TOPS, 4),
           "frac_mfma_i8_peak": round(tops / MFMA_I8_PEAK_TOPS, 4), "mean_launch_us": round(mean_ms * 1e3, 3),
           "weight_gbps": round(nbytes_w / (mean_ms * 1e-3) / 1e9, 1), "replicas": reps,
           "workspace_bytes": ws_bytes}
    del g, ws, w0, work
    torch.cuda.empty_cache()
    return res


GEMM_CASES = [("gguf:q4_k", 512), ("gguf:q8_0", 512), ("gguf:q6_k", 512), ("gguf:q4_0", 512), ("gguf:iq4_xs", 512),
              ("gguf:iq2_xxs", 512), ("gguf:q4_k", 16), ("gguf:q4_k", 64), ("gguf:q4_k", 2048)]


def gemm_cpu_baseline(synth, fmt="gguf:q4_k", shape=(14336, 4096), rows=7168, M=512, seed=0x6E7C8000):
    """The oracle's product (binary64) on the first `rows` weight rows with M
    activation rows, one thread."""
    import numpy as np
    import oracle
    N, K = shape
    _, B, S, _ = oracle.info(fmt)
    w = synth.payload(fmt, rows * K // B, seed, synth.binade(-6, -2, False))
    x = np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32)
    t0 = time.perf_counter()
    _, xq = oracle.quantize_q8_1(x)
    oracle.gemv_q8_1(fmt, w, rows, K, xq, M)
    secs = time.perf_counter() - t0
    return {"value": round(2.0 * M * rows * K / secs / 1e12, 6), "unit": "TOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{fmt} rows 0..{rows - 1} of [{N}, {K}] x {M} activation rows ({secs:.1f} s on one host core)"}


def gemm_only(torch, nq, synth, args):
    """The batched-product measurements alone (one JSON line): every GEMM_CASES
    entry at both shapes, the headline case's roofline, and the oracle beside it."""
    res = {}
    for fmt, M in product_cases(GEMM_CASES, args):
        for shape in product_shapes(args):
            key = f"gemm_q8_1 {fmt}{shape} M={M}"
            res[key] = gemm_measurement(torch, nq, synth, fmt, shape, M)
            log(f"{key}: {res[key]['tops']} TOP/s ({100 * res[key]['frac_alu_peak']:.1f}% of the ALU bound)")
    head = res.get("gemm_q8_1 gguf:q4_k[14336, 4096] M=512", next(iter(res.values())))
    roofline = {"bound": "alu", "achieved": head["tops"], "peak": round(GEMM_ALU_PEAK_TOPS, 1), "unit": "TOP/s",
                "frac": head["frac_alu_peak"], "traffic": None, "kernel": "k_gemm gguf:q4_k M=512",
                "mfma_i8_peak": MFMA_I8_PEAK_TOPS, "frac_mfma_i8_peak": head["frac_mfma_i8_peak"],
                "mean_launch_us": head["mean_launch_us"]}
    cpu = None if args.no_cpu_baseline else gemm_cpu_baseline(synth)
    line = {"metric": "gemm_q8_1 TOP/s (2 M N K per launch), 1\u00d7MI355X", "value": head["tops"], "unit": "TOP/s",
            "n_gpus": 1, "higher_is_better": True, "dtype": "i8xi8->i32, f32 scaling", "data": "synthetic",
            "config": {"workload": "q4_k weight [14336, 4096] x 512 q8_1 activation rows, rotating replicas"},
            "roofline": roofline, "cpu_baseline": cpu, "cases": res}
    print(json.dumps(line), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class pinned_to_one_core:
    """Run the enclosed code with this process's CPU affinity set to one core
    (the first it may use), restored afterwards."""

    def __enter__(self):
        self.before = os.sched_getaffinity(0)
        self.core = min(self.before)
        os.sched_setaffinity(0, {self.core})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.before)
        return False


def cpu_baseline(nq, synth, tensors, fraction=3):
    """The oracle on the first 1/fraction of every tensor's blocks, one thread
    pinned to one host core (payload generation, which is multithreaded, stays
    outside the timed calls)."""
    import numpy as np
    import oracle
    total_bytes = 0
    total_elems = 0
    secs = 0.0
    samples = []
    for name, fmt, shape, recipe, seed in tensors:
        _, B, S, T = oracle.info(fmt)
        nb = math.prod(shape) // B
        ns = max(1, nb // fraction)
        p = synth.payload(fmt, ns, seed, recipe)
        if T:
            p[-4:] = np.array([synth.divisor_bits(seed)], "<u4").view(np.uint8)
        samples.append((fmt, p, ns * B))
    with pinned_to_one_core() as pin:
        for fmt, p, n in samples:
            t0 = time.perf_counter()
            oracle.decode(fmt, p, [n], "bf16")
            secs += time.perf_counter() - t0
            total_bytes += p.size + n * 2
            total_elems += n
    return {"value": round(total_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first 1/{fraction} of the blocks of each of the {len(tensors)} tensors "
                      f"({total_elems / 1e9:.3f} G values to bf16, {secs:.1f} s on host core {pin.core})",
            "elements_per_s": round(total_elems / secs, 1), "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "affinity_before_pinning": len(pin.before), "pinned_core": pin.core}


def gemv_cpu_baseline(synth, fmt="gguf:q4_k", shape=(14336, 4096), rows=14336, seed=0x6E7C7000):
    """The oracle's product (binary64) on the first `rows` rows of one weight,
    M = 1, one thread."""
    import numpy as np
    import oracle
    N, K = shape
    _, B, S, _ = oracle.info(fmt)
    w = synth.payload(fmt, rows * K // B, seed, synth.binade(-6, -2, False))
    x = np.random.default_rng(seed).standard_normal((1, K)).astype(np.float32)
    t0 = time.perf_counter()
    _, xq = oracle.quantize_q8_1(x)
    oracle.gemv_q8_1(fmt, w, rows, K, xq, 1)
    secs = time.perf_counter() - t0
    nbytes = w.size + xq.size + 4 * rows
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{fmt} rows 0..{rows - 1} of [{N}, {K}], M = 1 ({secs:.1f} s on one host core)",
            "weights_per_s": round(rows * K / secs, 1)}


def product_cases(cases, args):
    """The (format, M) product cases to measure: all, or those --cases names."""
    if not args.cases:
        return cases
    want = [(c.rsplit(":", 1)[0], int(c.rsplit(":", 1)[1])) for c in args.cases.split(",")]
    return want


def product_shapes(args):
    """Weight shapes of the product measurements: both Llama-3-8B shapes, or --product-shapes."""
    if not args.product_shapes:
        return [[14336, 4096], [4096, 14336]]
    return [[int(v) for v in t.split("x")] for t in args.product_shapes.split(",")]


def gemv_only(torch, nq, synth, args):
    """The product measurements alone (one JSON line): every GEMV_CASES entry
    at both shapes, the dominant one's roofline, and the oracle beside it."""
    res = {}
    for fmt, M in product_cases(GEMV_CASES, args):
        for shape in product_shapes(args):
            key = f"gemv_q8_1 {fmt}{shape} M={M}"
            res[key] = gemv_measurement(torch, nq, synth, fmt, shape, M)
            log(f"{key}: {res[key]['gbps']} GB/s ({100 * res[key]['frac_hbm_peak']:.1f}% of peak)")
    head = res.get("gemv_q8_1 gguf:q4_k[14336, 4096] M=1", next(iter(res.values())))
    roofline = {"bound": "hbm", "achieved": head["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": head["frac_hbm_peak"], "traffic": None, "kernel": "gemv_q8_1 gguf:q4_k M=1 (k_gemv1)",
                "bytes_per_launch": head["bytes_per_launch"], "mean_launch_us": head["mean_launch_us"]}
    cpu = None if args.no_cpu_baseline else gemv_cpu_baseline(synth)
    line = {"metric": "gemv_q8_1 GB/s (weight + activation + output) per launch, 1\u00d7MI355X",
            "value": head["gbps"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "q4_k weight [14336, 4096] x one q8_1 activation row, rotating replicas"},
            "roofline": roofline, "cpu_baseline": cpu, "cases": res}
    print(json.dumps(line), flush=True)


def formats_only(torch, nq, synth, args):
    """Single-tensor decodes of the named formats at the named shapes, each
    over a cold rotation (rotating_measurement): one JSON line of its own.
    A small, fixed target for counter and trace runs.  It calls only
    nq_format_query and nq_dequantize_packed, so it also runs against earlier
    builds of the library."""
    from synth import workloads
    names = [f for f in args.formats.split(",") if f]
    shapes = [[int(d) for d in sh.split("x")] for sh in args.shapes.split(",") if sh]
    need = 0
    for f in names:
        info = nq.format_query(f)
        for sh in shapes:
            need = max(need, math.prod(sh) // info.block_values * info.block_bytes + info.trailer_bytes)
    staging = torch.empty(need, dtype=torch.uint8, pin_memory=True)
    res = {}
    for sh in shapes:
        for f in names:
            info = nq.format_query(f)
            key = f"{f}{sh}->{args.dtype}"
            res[key] = rotating_measurement(torch, nq, synth, key, f, sh, workloads.recipe_for(f), 0x6E718000 + info.id,
                                            args.dtype, staging, launches=args.launches)
            log(f"{key}: {res[key]['gbps']} GB/s ({100 * res[key]['frac_hbm_peak']:.1f}% of peak), "
                f"{res[key]['replicas']} replicas")
    print(json.dumps({"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "data": "synthetic",
                      "call": "nq_dequantize_packed, one tensor per launch", "workloads": res}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-per-format", action="store_true", help="skip the rotating per-workload timings")
    ap.add_argument("--gemv-only", action="store_true",
                    help="measure only the products with q8_1 activations (one JSON line of its own)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="measure only the batched products on the matrix cores (one JSON line of its own)")
    ap.add_argument("--cases", default="", metavar="FMT:M,...",
                    help="with --gemv-only / --gemm-only: measure only these (format, activation rows) cases")
    ap.add_argument("--product-shapes", default="", metavar="NxK,...",
                    help="with --gemv-only / --gemm-only: weight shapes (default [14336, 4096] and [4096, 14336])")
    ap.add_argument("--formats", default="", metavar="F1,F2,...",
                    help="measure only single-tensor decodes of these formats at --shapes (one JSON line of its own)")
    ap.add_argument("--shapes", default="14336x4096", metavar="RxC,...", help="shapes for --formats")
    ap.add_argument("--dtype", default="bf16", choices=sorted(OUT_CODES), help="output type for --formats")
    ap.add_argument("--launches", type=int, default=60, help="launches per timed replay for --formats")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="first run a plain device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode needs no collective and this build runs on a single "
              "MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_quantized_weight_nq_amd as nq
    import synth
    from synth import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nq.library()  # fails loudly if libnq.so is missing
    log(f"device {torch.cuda.get_device_name(0)}")

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.calibrate_copy} MiB device copies done")
        del a, b

    if args.formats:
        formats_only(torch, nq, synth, args)
        return
    if args.gemv_only:
        gemv_only(torch, nq, synth, args)
        return
    if args.gemm_only:
        gemm_only(torch, nq, synth, args)
        return

    tensors, _ = workloads.config5()
    staging = staging_buffer(torch, tensors, nq)
    t0 = time.perf_counter()
    items = [Tensor(n, f, s, r, sd, "bf16", staging, torch, nq, synth) for n, f, s, r, sd in tensors]
    torch.cuda.synchronize()
    log(f"generated and uploaded {len(items)} payloads in {time.perf_counter() - t0:.1f} s")
    step_bytes = sum(it.algo_bytes for it in items)
    payload_bytes = sum(it.nbytes for it in items)
    elems = sum(it.nelems for it in items)

    # the step: one many-tensor call (one launch per format here)
    call = nq.ManyCall([it.desc() for it in items], OUT_CODES["bf16"])
    eager_wall_ms, eager_event_ms = time_eager_many(torch, call, args.steps, args.warmup)
    log(f"eager step (one many-tensor call): wall {eager_wall_ms:.3f} ms, events {eager_event_ms:.3f} ms")
    step_graph = capture_many(torch, call)
    graph_ms, graph_wall_ms = time_graph(torch, step_graph, args.steps, warmup=args.warmup)
    log(f"graph step (one many-tensor call): events {graph_ms:.3f} ms, wall {graph_wall_ms:.3f} ms")
    del step_graph
    ms_per_step = graph_wall_ms
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the same step as 226 single-tensor calls
    pt_graph = capture(torch, nq, items)
    pt_ms, pt_wall_ms = time_graph(torch, pt_graph, args.steps, warmup=args.warmup)
    del pt_graph
    pt_eager_wall_ms, pt_eager_event_ms = time_eager(torch, nq, items, max(2, args.steps // 2), 1)
    log(f"graph step (226 single-tensor calls): events {pt_ms:.3f} ms, wall {pt_wall_ms:.3f} ms "
        f"({step_bytes / (pt_wall_ms * 1e-3) / 1e9:.1f} GB/s)")

    formats = per_format_times(torch, nq, items, reps=max(2, args.steps // 2))
    dom = max(formats, key=lambda f: formats[f]["total_ms"])
    d = formats[dom]
    achieved = d["bytes_per_launch"] / (d["mean_launch_us"] * 1e-6) / 1e9
    for f in formats.values():
        del f["total_ms"]
    del items, call
    torch.cuda.empty_cache()
    ceiling = stream_ceiling(torch, nq, d["read_bytes_per_launch"], d["bytes_per_launch"] - d["read_bytes_per_launch"],
                             launches=10)
    log(f"stream ceiling at {dom}'s read/write bytes: {ceiling['gbps']} GB/s")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": profiled_traffic(dom),
                "kernel": f"k_decode_many {dom} -> bf16 ({d['tensors']} tensors per launch)",
                "bytes_per_launch": d["bytes_per_launch"], "mean_launch_us": d["mean_launch_us"],
                "copy_ceiling": ceiling, "frac_of_copy_ceiling": round(achieved / ceiling["gbps"], 4)}

    extra = {}
    ceilings = {}
    if not args.no_per_format:
        # streaming ceilings at representative read:write mixes (bytes per value) and sizes (values)
        for key, (rb, wb, n) in {"1:1 copy": (1, 1, 58720256), "q4_k -> bf16": (0.5625, 2, 58720256),
                                 "q8_0 -> bf16": (1.0625, 2, 58720256), "iq2_xxs -> f32": (0.2578, 4, 58720256),
                                 "q4_k [4096, 4096] -> bf16": (0.5625, 2, 16777216),
                                 "q6_k [4096, 4096] -> bf16": (0.8203125, 2, 16777216)}.items():
            ceilings[key] = stream_ceiling(torch, nq, int(rb * n), int(wb * n))
            log(f"stream ceiling {key}: {ceilings[key]['gbps']} GB/s")
        # every format at the [14336, 4096] shape -> bf16
        st_all = torch.empty(14336 * 4096 // 256 * 292 + 4, dtype=torch.uint8, pin_memory=True)
        for fid in range(nq.format_count()):
            fmt = nq.format_by_id(fid).name.decode()
            key = f"all_formats {fmt}[14336, 4096]->bf16"
            extra[key] = rotating_measurement(torch, nq, synth, key, fmt, [14336, 4096], workloads.recipe_for(fmt),
                                              0x6E718000 + fid, "bf16", st_all)
            log(f"{key}: {extra[key]['gbps']} GB/s ({100 * extra[key]['frac_hbm_peak']:.1f}% of peak)")
        del st_all
        for cfg in (1, 2, 3, 4):
            ts, dtypes = workloads.CONFIGS[cfg]()
            st2 = staging_buffer(torch, ts, nq)
            for name, fmt, shape, recipe, seed in ts:
                for dt in dtypes:
                    key = f"{name}->{dt}"
                    extra[key] = rotating_measurement(torch, nq, synth, name, fmt, shape, recipe, seed, dt, st2)
                    if cfg == 1:
                        extra[key]["launch_bound"] = True
                        extra[key]["note"] = ("1.1-1.3 MB per launch: the launch's start-up and drain, not HBM, "
                                              "set its time")
                    log(f"{key}: {extra[key]['gbps']} GB/s ({100 * extra[key]['frac_hbm_peak']:.1f}% of peak)")
            del st2
        # nvfp4 planes stacked from two and eight sources (a gate/up pair, eight experts' slices)
        for shape, nd in (([2 * 14336, 4096], 2), ([8 * 1024, 4096], 8)):
            key = f"nvfp4x{nd}{shape}->bf16"
            st2 = torch.empty(math.prod(shape) // 64 * 36 + 4 * nd, dtype=torch.uint8, pin_memory=True)
            extra[key] = rotating_measurement(torch, nq, synth, key, "nvfp4", shape, workloads.recipe_for("nvfp4"),
                                              0x6E710000 + 77 * nd, "bf16", st2, divisors=nd)
            log(f"{key}: {extra[key]['gbps']} GB/s ({100 * extra[key]['frac_hbm_peak']:.1f}% of peak)")
            del st2
        for scheme, in_dtype in (("q4_g64_fp16", "bf16"), ("q8_g32_fp16", "f32")):
            key = f"grouped_absmax {in_dtype}->{scheme}[14336, 4096]"
            extra[key] = gq_measurement(torch, nq, scheme, [14336, 4096], in_dtype)
            log(f"{key}: {extra[key]['gbps']} GB/s ({100 * extra[key]['frac_hbm_peak']:.1f}% of peak)")
        for fmt in ("fp8_e4m3fn_row_bf16", "fp8_e4m3fn_row_fp16"):
            key = f"{fmt}[14336, 4096]->bf16"
            extra[key] = fp8_row_measurement(torch, nq, fmt, [14336, 4096], "bf16")
            log(f"{key}: {extra[key]['gbps']} GB/s ({100 * extra[key]['frac_hbm_peak']:.1f}% of peak)")
        # products with q8_1 activations: the decode-phase shapes of a Llama-3-8B layer
        for fmt, M in GEMV_CASES:
            for shape in ([14336, 4096], [4096, 14336]):
                key = f"gemv_q8_1 {fmt}{shape} M={M}"
                extra[key] = gemv_measurement(torch, nq, synth, fmt, shape, M)
                log(f"{key}: {extra[key]['gbps']} GB/s ({100 * extra[key]['frac_hbm_peak']:.1f}% of peak)")
        # batched products (prefill-like activation batches) on the matrix cores
        for fmt, M in GEMM_CASES:
            for shape in ([14336, 4096], [4096, 14336]):
                key = f"gemm_q8_1 {fmt}{shape} M={M}"
                extra[key] = gemm_measurement(torch, nq, synth, fmt, shape, M)
                log(f"{key}: {extra[key]['tops']} TOP/s ({100 * extra[key]['frac_alu_peak']:.1f}% of the ALU bound)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(nq, synth, tensors)
        log(f"cpu baseline: {cpu['value']} GB/s ({cpu['sample']}; {cpu['cpu_model']}, nproc {cpu['nproc']})")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3-8b weight set: 226 tensors, q4_k/q6_k/q8_0/nvfp4/tq2_0 rotation -> bf16",
                   "output_dtype": "bf16", "call": "one nq_dequantize_packed_many per step (one launch per format)",
                   "tensors": len(tensors), "elements": elems, "payload_bytes": payload_bytes,
                   "output_bytes": step_bytes - payload_bytes, "graph_event_ms_per_step": round(graph_ms, 4),
                   "eager_wall_ms_per_step": round(eager_wall_ms, 4), "eager_event_ms_per_step": round(eager_event_ms, 4),
                   "frac_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "single_tensor_calls": {
                       "launches_per_step": len(tensors), "graph_wall_ms_per_step": round(pt_wall_ms, 4),
                       "graph_event_ms_per_step": round(pt_ms, 4),
                       "eager_wall_ms_per_step": round(pt_eager_wall_ms, 4),
                       "eager_event_ms_per_step": round(pt_eager_event_ms, 4),
                       "gbps": round(step_bytes / (pt_wall_ms * 1e-3) / 1e9, 1)}},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_format": {"step": formats, "ceilings": ceilings, "workloads": extra},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
