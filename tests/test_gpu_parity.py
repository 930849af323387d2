"""GPU (gfx950) decode through the C ABI against the oracle, bit for bit.

Every comparison is exact except NaN payloads, which the DequantizePacked page
leaves unspecified (compared by class).  Inputs come from the seeded
generator; sizes span many workgroups with a ragged tail, and the full-size
workloads are compared in full, the weight-set workload through the
many-tensor call the benchmark times.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_nq_amd as nq
import compare
import oracle
import synth
from synth import workloads
from gpu_util import TORCH_DT, announce, decode, oracle_blocks, oracle_decode_parallel, oracle_threads, to_numpy, upload

pytestmark = pytest.mark.gpu

FORMATS = oracle.format_names()
RAW = synth.raw()
RECIPE = synth.binade(-12, -6, True)


def _check(fmt, payload, shape, dtype, **kw):
    got, _, _ = decode(fmt, payload, shape, dtype, **kw)
    ref = oracle.decode(fmt, payload, shape, dtype)
    assert compare.same(got, ref, dtype), f"{fmt} {shape} {dtype} {kw}: {compare.describe(got, ref, dtype)}"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_every_format_and_output_type(fmt, dtype):
    info = nq.format_query(fmt)
    nblocks = 2053  # several waves of workgroups and a ragged last iteration
    for r, recipe in enumerate([RAW if fmt != "nvfp4" else RECIPE, RECIPE]):
        announce(f"every_format {fmt} {dtype} recipe={recipe} blocks={nblocks}")
        p = synth.payload(fmt, nblocks, 500 + 7 * info.id + r, recipe)
        _check(fmt, p, [nblocks * info.block_values], dtype)


@pytest.mark.parametrize("fmt", ["gguf:q4_0", "gguf:mxfp4", "gguf:q6_k", "gguf:iq2_xs", "nvfp4", "gguf:tq1_0",
                                 "gguf:q3_k", "gguf:iq1_m"])
def test_payload_offsets_0_to_15(fmt):
    info = nq.format_query(fmt)
    nblocks = 301
    p = synth.payload(fmt, nblocks, 9, RECIPE)
    for off in range(16):
        announce(f"payload_offset {fmt} off={off}")
        _check(fmt, p, [nblocks * info.block_values], "bf16", pay_off=off)


@pytest.mark.parametrize("dtype,out_off", [("f32", 1), ("f32", 3), ("bf16", 1), ("bf16", 5), ("f16", 7),
                                           ("f64", 1)])
def test_unaligned_output_takes_scalar_stores(dtype, out_off):
    for fmt in ("gguf:q8_0", "gguf:q4_k", "gguf:iq3_s", "gguf:nvfp4"):
        info = nq.format_query(fmt)
        p = synth.payload(fmt, 129, 21, RECIPE)
        announce(f"unaligned_output {fmt} {dtype} out_off={out_off}")
        got, obuf, _ = decode(fmt, p, [129 * info.block_values], dtype, out_off=out_off)
        ref = oracle.decode(fmt, p, [129 * info.block_values], dtype)
        assert compare.same(got, ref, dtype), compare.describe(got, ref, dtype)
        head = to_numpy(obuf[:out_off], dtype)
        tail = to_numpy(obuf[out_off + got.size:], dtype)
        assert np.all(compare.nan_mask(head, dtype)) and np.all(compare.nan_mask(tail, dtype))


@pytest.mark.parametrize("shape", [[3, 2, 512], [1, 256], [256], [7, 1, 256]])
def test_shapes_are_flat_row_major(shape):
    for fmt in ("gguf:q2_k", "gguf:iq4_xs"):
        info = nq.format_query(fmt)
        nb = int(np.prod(shape)) // info.block_values
        p = synth.payload(fmt, nb, 3, RECIPE)
        announce(f"shape {fmt} {shape}")
        _check(fmt, p, shape, "f32")


def test_empty_tensors_launch_nothing():
    for fmt, shape in [("gguf:q4_k", [0, 256]), ("gguf:q8_0", [5, 0]), ("nvfp4", [0, 64]), ("gguf:mxfp4", [0])]:
        info = nq.format_query(fmt)
        p = synth.payload(fmt, 0, 1, RECIPE)
        announce(f"empty {fmt} {shape}")
        payload, _ = upload(p)
        sentinel = torch.full((8,), 7.0, device="cuda:0")
        out = torch.empty(0, device="cuda:0")
        y = nq.dequantize_packed(fmt, payload, shape, torch.float32, out=out)
        torch.cuda.synchronize()
        assert y.numel() == 0 and torch.all(sentinel == 7.0)


def test_metadata_errors_return_before_launch():
    fid = nq.format_query("gguf:q4_0").id
    p = synth.payload("gguf:q4_0", 4, 1, RECIPE)
    payload, _ = upload(p)
    out = torch.full((128,), 3.0, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    announce("metadata errors q4_0")
    cases = [([128], p.size - 1, 0, 6), ([4, 31], p.size, 0, 5), ([-1, 32], p.size, 0, 4), ([], p.size, 0, 3),
             ([128], p.size, 9, 8), ([128], p.size + 18, 0, 6)]
    for shape, nbytes, dt, want in cases:
        st = nq.dequantize_packed_raw(fid, payload.data_ptr(), nbytes, shape, dt, out.data_ptr(), stream)
        assert st == want, (shape, nbytes, dt, st)
    assert nq.dequantize_packed_raw(99, payload.data_ptr(), p.size, [128], 0, out.data_ptr(), stream) == 2
    assert nq.dequantize_packed_raw(fid, 0, p.size, [128], 0, out.data_ptr(), stream) == 1
    assert nq.dequantize_packed_raw(fid, payload.data_ptr(), p.size, [128], 0, 0, stream) == 1
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_mxfp4_every_exponent_byte_and_code():
    blocks = b"".join(bytes([e]) + bytes([c | ((15 - c) << 4) for c in range(16)]) for e in range(256))
    p = np.frombuffer(blocks, np.uint8)
    for dtype in ("f32", "bf16", "f16"):
        announce(f"mxfp4 exhaustive {dtype}")
        _check("gguf:mxfp4", p, [256 * 32], dtype)


def test_nvfp4_every_scale_byte_and_code():
    rows = []
    for e in range(256):
        rows.append(bytes([e, (e + 1) & 255, (e + 2) & 255, (e + 3) & 255]) +
                    bytes([c | ((15 - c) << 4) for c in range(8)] * 4))
    p = np.frombuffer(b"".join(rows), np.uint8)
    for dtype in ("f32", "bf16", "f16"):
        announce(f"gguf:nvfp4 exhaustive {dtype}")
        _check("gguf:nvfp4", p, [256 * 64], dtype)
        for d_w in (1.0, 3.0, 7.1234567, 448.0, 1e-30, 3e38, -3.0, -0.0, 0.0, float("inf"), float("-inf"),
                    float("nan"), 1e-40):
            announce(f"nvfp4 exhaustive {dtype} d_w={d_w}")
            q = np.concatenate([p, np.array([d_w], "<f4").view(np.uint8)])
            _check("nvfp4", q, [256 * 64], dtype)


def test_output_conversion_edges_through_q8_k():
    """y = d * q with binary32 d covering every high half-word with the low
    half-words the oracle's conversion pin uses (at and around the bf16 and f16
    rounding points, odd-LSB ties and f16's subnormal tie points included) plus
    2^18 random words:
    exercises the hardware bf16/f16 conversions on ties, subnormals, overflow
    and NaN (q = 1 converts d itself; the other codes scale it)."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x2FFF, 0x3000,
                     0x3001, 0x3FFF, 0x4000, 0x4001, 0x5FFF, 0x6000, 0x6001, 0x7FFF, 0x8000, 0x8001,
                     0xBFFF, 0xC000, 0xC001, 0xFFFF], dtype=np.uint32)
    rand = np.random.default_rng(2025).integers(0, 2 ** 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    d = np.concatenate([(hi[:, None] | lows[None, :]).ravel(), rand])
    n = d.size
    blk = np.zeros((n, 292), dtype=np.uint8)
    blk[:, 0:4] = d.view(np.uint8).reshape(n, 4)
    q = np.array([1, -1, 2, 3, -128, 127, 0, 5] * 32, dtype=np.int8)
    blk[:, 4:260] = q.view(np.uint8)
    p = blk.ravel()
    for dtype in ("bf16", "f16", "f32"):
        announce(f"q8_k conversion edges {dtype} blocks={n}")
        _check("gguf:q8_k", p, [n * 256], dtype)


def test_side_stream_is_ordered():
    fmt = "gguf:q4_k"
    p = synth.payload(fmt, 4096, 8, RECIPE)
    payload, _ = upload(p)
    s = torch.cuda.Stream()
    announce("side stream q4_k")
    with torch.cuda.stream(s):
        out = torch.empty(4096 * 256, dtype=torch.bfloat16, device="cuda:0")
        nq.dequantize_packed(fmt, payload, [4096, 256], torch.bfloat16, out=out, stream=s)
    s.synchronize()
    ref = oracle.decode(fmt, p, [4096 * 256], "bf16")
    assert compare.same(to_numpy(out, "bf16"), ref, "bf16")


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q8_0", "nvfp4", "gguf:iq2_xxs", "gguf:tq1_0", "gguf:mxfp4",
                                 "gguf:q3_k", "gguf:iq4_nl", "gguf:iq1_m", "gguf:iq2_s"])
def test_every_tile_size_class(fmt):
    """Launch sizes that take each of the launcher's tile sizes (units per
    resident workgroup q, 8 resident per compute unit: 100 -> 1, 200 -> 2,
    600 -> 4, 1500 -> 8, 2100 -> the format's long-launch size; the IQ
    formats with large codebooks step up by q alone, to 16 at 3100), each one block past a
    whole number of units per workgroup, to f32 and bf16, compared in full."""
    info = nq.format_query(fmt)
    B = info.block_values
    resident = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    qs = (100, 200, 400, 800, 1500, 2100, 3100) if fmt in ("gguf:iq1_m", "gguf:iq2_s") else (100, 200, 600, 1500, 2100)
    for q in qs:
        n = resident * q * 8 + B
        nb = n // B
        p = synth.payload(fmt, nb, 40 + q, RECIPE)
        for dtype in ("f32", "bf16"):
            announce(f"tile_size_class {fmt} q={q} blocks={nb} {dtype}")
            _check(fmt, p, [n], dtype)


# ---------------------------------------------------------------------------
# Full-size workloads, compared in full against the oracle, whose decode is
# fanned out over host threads (gpu_util.oracle_threads: the cores this
# process may use, at most 16).
# ---------------------------------------------------------------------------
def _full_size(name, fmt, shape, recipe, seed, dtype):
    info = nq.format_query(fmt)
    nb = int(np.prod(shape)) // info.block_values
    announce(f"full-size {name} {fmt} {shape} {dtype} seed={seed:#x} threads={oracle_threads()}")
    p = synth.payload(fmt, nb, seed, recipe)
    payload, _ = upload(p)
    out = nq.dequantize_packed(fmt, payload, shape, TORCH_DT[dtype])
    torch.cuda.synchronize()
    got = to_numpy(out.reshape(-1), dtype)
    del out, payload
    ref = oracle_decode_parallel(fmt, p, nb, dtype)
    assert compare.same(got, ref, dtype), f"{name}: {compare.describe(got, ref, dtype)}"
    torch.cuda.empty_cache()


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_full_size_configs_in_full(config):
    tensors, dtypes = workloads.CONFIGS[config]()
    for name, fmt, shape, recipe, seed in tensors:
        for dtype in dtypes:
            _full_size(name, fmt, shape, recipe, seed, dtype)


def test_full_size_llama3_8b_set_in_full():
    """The whole Llama-3-8B-shaped set (226 tensors, 8.03 G values) decoded to
    bf16 by one nq_dequantize_packed_many call, the launch configuration the
    benchmark times, and every output compared with the oracle."""
    tensors, _ = workloads.config5()
    items = []
    for name, fmt, shape, recipe, seed in tensors:
        info = nq.format_query(fmt)
        nb = int(np.prod(shape)) // info.block_values
        p = synth.payload(fmt, nb, seed, recipe)
        payload = torch.from_numpy(p).to("cuda:0")
        out = torch.empty(int(np.prod(shape)), dtype=torch.bfloat16, device="cuda:0")
        items.append((name, fmt, shape, recipe, seed, nb, info.id, payload, out))
        del p
    announce(f"full-size llama3-8b set: one many-tensor call over {len(items)} tensors")
    st, failed = nq.dequantize_packed_many_raw([(it[6], it[7].data_ptr(), it[7].numel(), it[2], it[8].data_ptr())
                                                 for it in items], 2, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (st, failed) == (0, -1)
    threads = oracle_threads()
    for k, (name, fmt, shape, recipe, seed, nb, fid, payload, out) in enumerate(items):
        if k % 20 == 0:
            announce(f"full-size llama3-8b set: comparing tensor {k} ({name}), oracle on {threads} threads")
        got = to_numpy(out, "bf16")
        ref = oracle_decode_parallel(fmt, synth.payload(fmt, nb, seed, recipe), nb, "bf16", threads)
        assert compare.same(got, ref, "bf16"), f"{name}: {compare.describe(got, ref, 'bf16')}"
    del items
    torch.cuda.empty_cache()


def test_graph_replays_match_eager():
    """Decodes captured in a HIP graph give the eager result on every replay,
    with eager work, output clearing and synchronization between replays."""
    cases = [("gguf:q4_k", 512), ("nvfp4", 777), ("gguf:iq2_xxs", 300), ("gguf:q6_k", 129)]
    items = []
    for fmt, nb in cases:
        info = nq.format_query(fmt)
        p = synth.payload(fmt, nb, 31, RECIPE)
        payload, keep = upload(p)
        n = nb * info.block_values
        ref = nq.dequantize_packed(fmt, payload, [n], torch.bfloat16)
        out = torch.zeros(n, dtype=torch.bfloat16, device="cuda:0")
        items.append((fmt, payload, keep, n, ref, out, p))
    torch.cuda.synchronize()
    for fmt, _, _, n, ref, _, p in items:
        assert compare.same(to_numpy(ref, "bf16"), oracle.decode(fmt, p, [n], "bf16"), "bf16")
    announce("graph capture of 4 decodes")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for fmt, payload, _, n, _, out, _ in items:
            st = nq.dequantize_packed_raw(nq.format_query(fmt).id, payload.data_ptr(), payload.numel(), [n], 2,
                                          out.data_ptr(), h)
            assert st == 0
    other = synth.payload("gguf:q8_0", 1000, 5, RECIPE)
    other_dev, _ = upload(other)
    for r in range(4):
        announce(f"graph replay {r}")
        for *_, out, _ in items:
            out.zero_()
        nq.dequantize_packed("gguf:q8_0", other_dev, [32000], torch.float32)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for fmt, _, _, n, ref, out, _ in items:
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (fmt, r)


# ---------------------------------------------------------------------------
# nvfp4 planes stacked from several sources (one divisor per source).
# ---------------------------------------------------------------------------
def _stacked_check(shape, divisors, dtype, seed, pay_off=0, d_ws=None):
    N = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    nb = N * shape[-1] // 64
    p = synth.payload("nvfp4", nb, seed, workloads.recipe_for("nvfp4"), divisor=d_ws, divisors=divisors)
    payload, _keep = upload(p, pay_off)
    out = nq.dequantize_nvfp4_stacked(payload, shape, divisors, TORCH_DT[dtype])
    torch.cuda.synchronize()
    got = to_numpy(out.reshape(-1), dtype)
    ref = oracle.decode_nvfp4_stacked(p, shape, divisors, dtype)
    assert compare.same(got, ref, dtype), f"{shape} D={divisors} {dtype} off={pay_off}: {compare.describe(got, ref, dtype)}"


@pytest.mark.parametrize("shape,divisors", [([24, 128], 1), ([24, 128], 2), ([24, 128], 3), ([24, 128], 24),
                                            ([40, 64], 40), ([40, 64], 8), ([6, 4096], 3), ([96, 512], 4),
                                            ([3, 8, 1024], 6), ([4100, 64], 4100), ([2050, 128], 5)])
def test_nvfp4_stacked_divisors(shape, divisors):
    for dtype in ("f32", "bf16", "f16", "f64"):
        for off in (0, 1, 2, 3):
            announce(f"nvfp4_stacked {shape} D={divisors} {dtype} off={off}")
            _stacked_check(shape, divisors, dtype, 70 + divisors, pay_off=off)


def test_nvfp4_stacked_full_size_sources():
    """Stacked gate/up and q/k/v-like planes at Llama-3-8B sizes, compared in full."""
    for shape, divisors in (([2 * 14336, 4096], 2), ([3 * 4096, 4096], 3), ([8 * 1024, 4096], 8)):
        announce(f"nvfp4_stacked full size {shape} D={divisors}")
        _stacked_check(shape, divisors, "bf16", 5 + divisors)


def test_nvfp4_stacked_one_divisor_is_plain_nvfp4():
    p = synth.payload("nvfp4", 4000, 17, workloads.recipe_for("nvfp4"))
    payload, _keep = upload(p)
    a = nq.dequantize_nvfp4_stacked(payload, [1000, 256], 1, torch.bfloat16)
    b = nq.dequantize_packed("nvfp4", payload, [1000, 256], torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# Row-scaled FP8: fp8_e4m3fn_row_bf16 / fp8_e4m3fn_row_fp16.
# ---------------------------------------------------------------------------
def _fp8_payload(N, K, seed, scale_words=None):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=N * K, dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=N, dtype=np.uint16) if scale_words is None else scale_words
    return np.concatenate([codes, np.asarray(scales, np.uint16).astype("<u2").view(np.uint8)])


def _fp8_check(fmt, p, shape, dtype, pay_off=0, out_off=0):
    payload, _keep = upload(p, pay_off)
    n = shape[0] * shape[1]
    obuf = torch.full((n + out_off + 8,), float("nan"), dtype=TORCH_DT[dtype], device="cuda:0")
    out = obuf[out_off:out_off + n]
    nq.dequantize_fp8_row(fmt, payload, shape, TORCH_DT[dtype], out=out)
    torch.cuda.synchronize()
    got = to_numpy(out, dtype)
    ref = oracle.decode_fp8_row(fmt, p, shape, dtype)
    assert compare.same(got, ref, dtype), f"{fmt} {shape} {dtype}: {compare.describe(got, ref, dtype)}"
    # the NaN fill around the output is untouched
    assert bool(torch.isnan(obuf[:out_off]).all()) and bool(torch.isnan(obuf[out_off + n:]).all())


@pytest.mark.parametrize("fmt", ["fp8_e4m3fn_row_bf16", "fp8_e4m3fn_row_fp16"])
@pytest.mark.parametrize("shape", [[7, 48], [5, 33], [3, 1], [1, 4099], [9, 7], [300, 4096], [1025, 96], [2, 70001]])
def test_fp8_row_every_output_type(fmt, shape):
    """Random code and scale words (NaN and infinite ones included, compared
    by class), rows shorter and longer than a thread's 16 values."""
    p = _fp8_payload(shape[0], shape[1], shape[0] * 31 + shape[1])
    for dtype in ("f32", "f16", "bf16", "f64"):
        announce(f"fp8_row {fmt} {shape} {dtype}")
        _fp8_check(fmt, p, shape, dtype)


@pytest.mark.parametrize("fmt", ["fp8_e4m3fn_row_bf16", "fp8_e4m3fn_row_fp16"])
def test_fp8_row_payload_and_output_offsets(fmt):
    p = _fp8_payload(37, 200, 5)
    for off in range(8):
        for dtype, out_off in (("bf16", off), ("f32", off % 4)):
            announce(f"fp8_row offsets {fmt} pay_off={off} {dtype} out_off={out_off}")
            _fp8_check(fmt, p, [37, 200], dtype, pay_off=off, out_off=out_off)


def test_fp8_row_full_size():
    """[14336, 4096] with valid scale words (positive finite), compared in full."""
    rng = np.random.default_rng(9)
    bf = (rng.integers(0x3B00, 0x3D00, size=14336)).astype(np.uint16)        # bfloat16 in [2^-9, 2^-5)
    f16 = (rng.integers(0x1C00, 0x2C00, size=14336)).astype(np.uint16)       # binary16 in [2^-8, 2^-4)
    for fmt, sw in (("fp8_e4m3fn_row_bf16", bf), ("fp8_e4m3fn_row_fp16", f16)):
        announce(f"fp8_row full size {fmt}")
        _fp8_check(fmt, _fp8_payload(14336, 4096, 11, sw), [14336, 4096], "bf16")


# ---------------------------------------------------------------------------
# grouped_absmax encoder (q4/q5/q6_g64_fp16, q8_g32_fp16).
# ---------------------------------------------------------------------------
_GQ_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}


def _gq_case(scheme, N, K, in_dtype, seed, x_off=0, c_off=0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-30, 10, (N, 1)))).astype(np.float32)
    x[0, : min(K, 40)] = 0.0
    t = torch.from_numpy(x).to(_GQ_TORCH[in_dtype])
    ox = t.view(torch.int16).numpy().view(np.uint16) if in_dtype in ("f16", "bf16") else t.numpy()
    st, wc, ws = oracle.grouped_absmax(scheme, ox, in_dtype)
    assert st == 0
    sid, G = nq.GQ_SCHEMES[scheme]
    # place the source and the codes at the requested offsets of larger buffers
    xb = torch.zeros(N * K + 16, dtype=t.dtype, device="cuda:0")
    xb[x_off:x_off + N * K].copy_(t.reshape(-1))
    cb = torch.full((N * K + 64,), 0x5A, dtype=torch.int8, device="cuda:0")
    ng = (K + G - 1) // G
    sb = torch.full((N * ng + 8,), 0x5A5A, dtype=torch.int16, device="cuda:0")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    h = torch.cuda.current_stream().cuda_stream
    rc = nq.quantize_grouped_absmax_raw(sid, xb.data_ptr() + x_off * xb.element_size(), [N, K],
                                        nq.DTYPE_CODES[in_dtype], cb.data_ptr() + c_off, sb.data_ptr(),
                                        status.data_ptr(), h)
    assert rc == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got_c = cb[c_off:c_off + N * K].cpu().numpy().reshape(N, K)
    got_s = sb[:N * ng].cpu().numpy().view(np.uint16).reshape(N, ng)
    assert np.array_equal(got_c, wc), f"{scheme} {N}x{K} {in_dtype} codes differ at {np.argwhere(got_c != wc)[:4]}"
    assert np.array_equal(got_s, ws), f"{scheme} {N}x{K} {in_dtype} scales differ"
    assert bool((cb[:c_off] == 0x5A).all()) and bool((cb[c_off + N * K:] == 0x5A).all())
    assert bool((sb[N * ng:] == 0x5A5A).all())


@pytest.mark.parametrize("scheme", ["q4_g64_fp16", "q5_g64_fp16", "q6_g64_fp16", "q8_g32_fp16"])
@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16", "f64"])
def test_grouped_absmax_matches_oracle(scheme, in_dtype):
    G = nq.GQ_SCHEMES[scheme][1]
    for N, K, x_off, c_off in ((33, 4 * G, 0, 0), (7, 3 * G + 24, 0, 0), (5, 70, 1, 3), (9, 13, 0, 1),
                               (3, 5, 2, 0), (257, 2 * G + 3, 0, 0), (64, 1024, 3, 2)):
        announce(f"grouped_absmax {scheme} {in_dtype} {N}x{K} x_off={x_off} c_off={c_off}")
        _gq_case(scheme, N, K, in_dtype, N * 7 + K, x_off, c_off)


def test_grouped_absmax_full_size():
    for scheme, in_dtype in (("q4_g64_fp16", "bf16"), ("q8_g32_fp16", "f32")):
        announce(f"grouped_absmax full size {scheme} {in_dtype} [4096, 4096]")
        _gq_case(scheme, 4096, 4096, in_dtype, 99)


def test_grouped_absmax_failures_and_status_reset():
    """Encoder failures set the status bits; the next call clears them."""
    x = torch.ones((3, 64), dtype=torch.float32, device="cuda:0")
    x[1, 5] = float("inf")
    x[2, 9] = 8321040.0  # q8: raw scale 65520 rounds to binary16 infinity
    announce("grouped_absmax failures")
    _, _, status = nq.quantize_grouped_absmax("q8_g32_fp16", x, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 3
    with pytest.raises(ValueError):
        nq.quantize_grouped_absmax("q8_g32_fp16", x)
    y = torch.ones((3, 64), dtype=torch.float32, device="cuda:0")
    codes, scales, status = nq.quantize_grouped_absmax("q8_g32_fp16", y)
    assert int(status.item()) == 0 and bool((codes == 127).all())
