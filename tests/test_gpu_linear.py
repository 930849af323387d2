"""GPU (gfx950) products with q8_1 activations through the C ABI, against the oracle.

The q8_1 quantizer is integer / byte work and must match the oracle bit for
bit.  The product's accumulation order is the kernel's, so it must meet the
oracle's criterion (tests/linear_criterion.py); repeated calls must agree bit
for bit.  Sizes span many workgroups with ragged row counts; the full-size
weights are checked on sampled rows in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_nq_amd as nq
import oracle
import synth
from gpu_util import announce, upload
from linear_criterion import check as linear_check

pytestmark = pytest.mark.gpu

GGUF = [f for f in oracle.format_names() if f.startswith("gguf:")]
TORCH_IN = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}


def _act(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * 2.0
    x[:, rng.integers(0, K, size=max(1, K // 61))] *= 30.0
    return x


def _source(x, in_dtype):
    """(oracle source array, torch CPU tensor of the same words)."""
    if in_dtype == "f32":
        xs = x.astype(np.float32)
        return xs, torch.from_numpy(xs)
    if in_dtype == "f64":
        return x, torch.from_numpy(x.copy())
    if in_dtype == "f16":
        xs = x.astype(np.float16).view(np.uint16)
        return xs, torch.from_numpy(xs.view(np.int16).copy()).view(torch.float16)
    xs = oracle.convert(x.astype(np.float32), "bf16").reshape(x.shape)
    return xs, torch.from_numpy(xs.view(np.int16).copy()).view(torch.bfloat16)


def _device_x(t, elem_off):
    """t on cuda:0 at element offset elem_off of its allocation."""
    buf = torch.zeros(t.numel() + elem_off + 8, dtype=t.dtype, device="cuda:0")
    view = buf[elem_off:elem_off + t.numel()].view(t.shape)
    view.copy_(t.to("cuda:0"))
    return view, buf


def _blocks_np(b):
    return b.cpu().numpy()


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16", "f64"])
@pytest.mark.parametrize("shape", [[3, 352], [5, 4096], [1, 14336], [8, 11008]])
def test_quantize_q8_1_matches_oracle(in_dtype, shape):
    M, K = shape
    x = _act(M, K, 17 * M + K)
    x[0, 64:96] = 0.0                   # an all-zero block
    x[-1, 32] = 1e-30                   # a block of tiny values
    x[-1, 96:128] = 65024.0             # a block whose sum overflows binary16
    xs, xt = _source(x, in_dtype)
    ost, ob = oracle.quantize_q8_1(xs, in_dtype)
    for off in (0, 1, 3):               # 16-byte aligned, then element offsets
        announce(f"quantize_q8_1 {in_dtype} {shape} off={off}")
        xd, _keep = _device_x(xt, off)
        blocks, status = nq.quantize_q8_1(xd, check=False)
        torch.cuda.synchronize()
        assert int(status.item()) == ost
        assert np.array_equal(_blocks_np(blocks), ob), f"{in_dtype} {shape} off={off}"


def test_quantize_q8_1_failures_and_status_reset():
    x = _act(2, 128, 5).astype(np.float32)
    x[0, 3] = np.nan
    x[1, 70] = 2.0 ** 23
    ost, ob = oracle.quantize_q8_1(x)
    announce("quantize_q8_1 failures")
    blocks, status = nq.quantize_q8_1(torch.from_numpy(x).cuda(), check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == ost == 3
    assert np.array_equal(_blocks_np(blocks), ob)
    with pytest.raises(ValueError):
        nq.quantize_q8_1(torch.from_numpy(x).cuda())
    # the status word is cleared by every call
    good = _act(2, 128, 6).astype(np.float32)
    blocks, status = nq.quantize_q8_1(torch.from_numpy(good).cuda(), check=True)
    assert int(status.item()) == 0


def _gemv(fmt, w_np, N, K, xq_np, w_off=0, stream=None):
    w, _keep = upload(w_np, w_off)
    xq = torch.from_numpy(np.ascontiguousarray(xq_np)).cuda()
    y = nq.gemv_q8_1(fmt, w, N, K, xq, stream=stream)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _weights(fmt, N, K, seed):
    _, B, _, _ = oracle.info(fmt)
    return synth.payload(fmt, N * K // B, seed, synth.binade(-6, -2, fmt in ("gguf:q4_0", "gguf:q8_0")))


@pytest.mark.parametrize("M", [1, 2, 3, 8])
@pytest.mark.parametrize("fmt", GGUF)
def test_gemv_every_format(fmt, M):
    _, B, _, _ = oracle.info(fmt)
    N, K = 37, 3 * max(B, 256)          # ragged against the rows a workgroup takes
    w = _weights(fmt, N, K, 300 + M)
    _, xq = oracle.quantize_q8_1(_act(M, K, M).astype(np.float32))
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    for w_off in (0, 1, 3):
        announce(f"gemv {fmt} N={N} K={K} M={M} w_off={w_off}")
        y = _gemv(fmt, w, N, K, xq, w_off)
        linear_check(y, ref, env, K, f"{fmt} M={M} w_off={w_off}")


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:iq2_xxs", "gguf:q8_0"])
def test_gemv_repeats_bit_for_bit_and_on_a_side_stream(fmt):
    N, K, M = 300, 4096, 2
    w = _weights(fmt, N, K, 8)
    _, xq = oracle.quantize_q8_1(_act(M, K, 9).astype(np.float32))
    announce(f"gemv repeat {fmt}")
    a = _gemv(fmt, w, N, K, xq)
    b = _gemv(fmt, w, N, K, xq)
    s = torch.cuda.Stream()
    c = _gemv(fmt, w, N, K, xq, stream=s)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_gemv_codebook_formats_loop_over_rows():
    """Codebook formats cap the grid at the resident workgroups and loop; a
    weight with more rows than that covers the loop."""
    fmt, N, K, M = "gguf:iq2_xxs", 40000, 256, 1
    w = _weights(fmt, N, K, 4)
    _, xq = oracle.quantize_q8_1(_act(M, K, 4).astype(np.float32))
    announce(f"gemv {fmt} N={N}")
    y = _gemv(fmt, w, N, K, xq)
    rows = np.r_[0:64, 16380:16400, N - 64:N]
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(y[:, rows], ref, env, K, fmt)


FULL = [("gguf:q4_k", 14336, 4096), ("gguf:q6_k", 4096, 14336), ("gguf:q8_0", 4096, 4096),
        ("gguf:tq2_0", 1024, 4096), ("gguf:iq2_xxs", 14336, 4096), ("gguf:iq4_xs", 4096, 14336),
        ("gguf:mxfp4", 14336, 4096), ("gguf:q5_k", 4096, 4096)]


@pytest.mark.parametrize("fmt,N,K,M", [f + (1,) for f in FULL] +
                         [("gguf:q4_k", 14336, 4096, 8), ("gguf:q4_0", 14336, 4096, 4),
                          ("gguf:iq2_xs", 4096, 14336, 2), ("gguf:q6_k", 1024, 14336, 8)])
def test_gemv_full_size_sampled_rows(fmt, N, K, M):
    """Llama-3-8B-shaped weights, M = 1 (the benchmark's launch) and a few
    decode batches: every output computed on the GPU, sampled rows against
    the oracle.  Single-round launches with one, two and three rows per
    chunk and the chunk loop (q6_k at [4096, 14336]) are among them."""
    w = _weights(fmt, N, K, 77)
    _, xq = oracle.quantize_q8_1(_act(M, K, 1).astype(np.float32))
    announce(f"gemv full {fmt} [{N}, {K}] M={M}")
    y = _gemv(fmt, w, N, K, xq)
    rng = np.random.default_rng(N + K)
    rows = np.unique(np.r_[0, 1, N - 1, rng.integers(0, N, size=61)])
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(y[:, rows], ref, env, K, fmt)
    assert np.all(np.isfinite(y))


def test_gemv_metadata_errors():
    w = torch.zeros(34 * 4, dtype=torch.uint8, device="cuda:0")
    xq = torch.zeros(36, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(nq.NqError):
        nq.gemv_q8_1("nvfp4", w, 1, 64, torch.zeros(72, dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(nq.NqError):
        nq.gemv_q8_1("gguf:q8_0", w[:33], 1, 32, xq)       # payload short
    with pytest.raises(nq.NqError):                        # nine activation rows
        nq.gemv_q8_1("gguf:q8_0", w[:34], 1, 32, torch.zeros(36 * 9, dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(nq.NqError):
        nq.gemv_q8_1("gguf:q4_k", w, 1, 32, xq)            # K not a multiple of 256


@pytest.mark.parametrize("fmt,K", [("gguf:q8_0", 16384), ("gguf:q4_k", 28672), ("gguf:q6_k", 16384),
                                   ("gguf:q4_1", 24576), ("gguf:iq4_xs", 24576)])
def test_gemv_rows_staged_in_chunks(fmt, K):
    """Rows longer than one staged chunk (12 KiB) are staged chunk by chunk."""
    N, M = 21, 2
    w = _weights(fmt, N, K, 12)
    _, xq = oracle.quantize_q8_1(_act(M, K, 12).astype(np.float32))
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    announce(f"gemv chunked {fmt} K={K}")
    y = _gemv(fmt, w, N, K, xq, 2)
    linear_check(y, ref, env, K, fmt)


@pytest.mark.parametrize("fmt,K", [("gguf:q8_0", 160), ("gguf:q4_0", 96), ("gguf:mxfp4", 288), ("gguf:nvfp4", 192)])
def test_gemv_k_not_a_multiple_of_128(fmt, K):
    """Other K take the activation's plain LDS layout."""
    N, M = 300, 3
    w = _weights(fmt, N, K, 31)
    _, xq = oracle.quantize_q8_1(_act(M, K, 31).astype(np.float32))
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    announce(f"gemv {fmt} K={K}")
    y = _gemv(fmt, w, N, K, xq, 1)
    linear_check(y, ref, env, K, fmt)


# --------------------------------------------------------------------------
# Batched products (any number of activation rows; more than 8 on the matrix
# cores, tq1_0 through the single-row kernel 8 rows at a time).
# --------------------------------------------------------------------------
def _gemm(fmt, w_np, N, K, xq_np, w_off=0, stream=None, split=True):
    w, _keep = upload(w_np, w_off)
    xq = torch.from_numpy(np.ascontiguousarray(xq_np)).cuda()
    y = nq.gemm_q8_1(fmt, w, N, K, xq, stream=stream, split=split)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _gemm_k(B):
    """K that leaves a partial last K step (256 values) where the block size allows."""
    return 352 if B == 32 else 384 if B in (64, 128) else 768


@pytest.mark.parametrize("fmt", GGUF)
def test_gemm_every_format(fmt):
    _, B, _, _ = oracle.info(fmt)
    K = _gemm_k(B)
    for N, M, w_off in [(300, 70, 0), (37, 9, 1), (129, 130, 3), (150, 5, 2)]:
        w = _weights(fmt, N, K, 400 + M)
        _, xq = oracle.quantize_q8_1(_act(M, K, M).astype(np.float32))
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        announce(f"gemm {fmt} N={N} K={K} M={M} w_off={w_off}")
        y = _gemm(fmt, w, N, K, xq, w_off)
        linear_check(y, ref, env, K, f"{fmt} N={N} M={M} w_off={w_off}")


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:iq3_s", "gguf:q5_0", "gguf:tq1_0"])
def test_gemm_up_to_4_rows_is_the_single_row_product(fmt):
    _, B, _, _ = oracle.info(fmt)
    N, K = 77, 2 * max(B, 256)
    w = _weights(fmt, N, K, 5)
    for M in (1, 3, 4):
        _, xq = oracle.quantize_q8_1(_act(M, K, 40 + M).astype(np.float32))
        announce(f"gemm vs gemv {fmt} M={M}")
        a = _gemm(fmt, w, N, K, xq)
        b = _gemv(fmt, w, N, K, xq)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q6_k", "gguf:iq2_xxs", "gguf:q4_1"])
def test_gemm_repeats_bit_for_bit_and_on_a_side_stream(fmt):
    N, K, M = 300, 1024, 100
    w = _weights(fmt, N, K, 8)
    _, xq = oracle.quantize_q8_1(_act(M, K, 9).astype(np.float32))
    announce(f"gemm repeat {fmt}")
    a = _gemm(fmt, w, N, K, xq)
    b = _gemm(fmt, w, N, K, xq)
    c = _gemm(fmt, w, N, K, xq, stream=torch.cuda.Stream())
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


GEMM_FULL = [("gguf:q4_k", 14336, 4096, 512), ("gguf:q8_0", 4096, 14336, 512), ("gguf:q6_k", 4096, 4096, 200),
             ("gguf:iq4_xs", 14336, 4096, 64), ("gguf:iq2_xxs", 4096, 4096, 100), ("gguf:q2_k", 1024, 14336, 72),
             ("gguf:q4_k", 4096, 14336, 64), ("gguf:q6_k", 14336, 4096, 320)]


@pytest.mark.parametrize("fmt,N,K,M", GEMM_FULL)
def test_gemm_full_size_sampled_rows(fmt, N, K, M):
    """Llama-3-8B-shaped weights with a batch of activation rows: every output
    computed on the GPU, sampled weight rows (all activation rows) against the
    oracle."""
    w = _weights(fmt, N, K, 78)
    _, xq = oracle.quantize_q8_1(_act(M, K, 2).astype(np.float32))
    announce(f"gemm full {fmt} [{N}, {K}] x {M}")
    y = _gemm(fmt, w, N, K, xq)
    rng = np.random.default_rng(N + K + M)
    rows = np.unique(np.r_[0, 127, 128, N - 1, rng.integers(0, N, size=36)])
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(y[:, rows], ref, env, K, fmt)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("fmt", GGUF)
def test_gemm_four_span_k_steps(fmt):
    """A grid of more than two 64-row tiles per compute unit (96 weight tiles
    by 9 activation tiles, the last one 8 rows; K ragged against the 4-span
    step where the block size allows) takes K steps of 128 values on a
    256-compute-unit device, with the weight rewritten once (workspace) or
    per tile (none): the same bits both ways, and sampled weight rows,
    every activation row, against the oracle."""
    _, B, _, _ = oracle.info(fmt)
    N, K, M = 12288, _gemm_k(B), 520
    w = _weights(fmt, N, K, 93)
    _, xq = oracle.quantize_q8_1(_act(M, K, 94).astype(np.float32))
    announce(f"gemm 4-span steps {fmt} [{N}, {K}] x {M}")
    y = _gemm(fmt, w, N, K, xq, w_off=1, split=True)
    y2 = _gemm(fmt, w, N, K, xq, w_off=1, split=False)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    rows = np.unique(np.r_[0, 127, 128, N - 1, np.random.default_rng(K).integers(0, N, size=28)])
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(y[:, rows], ref, env, K, f"{fmt} 4-span steps")
    assert np.all(np.isfinite(y))


def test_gemm_metadata_errors():
    w = torch.zeros(34 * 4, dtype=torch.uint8, device="cuda:0")
    xq = torch.zeros(36 * 9, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(nq.NqError):
        nq.gemm_q8_1("nvfp4", w, 1, 64, torch.zeros(72 * 9, dtype=torch.uint8, device="cuda:0"))
    with pytest.raises(nq.NqError):
        nq.gemm_q8_1("gguf:q8_0", w[:33], 1, 32, xq)       # payload short
    with pytest.raises(nq.NqError):
        nq.gemm_q8_1("gguf:q4_k", w, 1, 32, xq)            # K not a multiple of 256


@pytest.mark.parametrize("fmt,N,K,M", [("gguf:q4_k", 4096, 14336, 64), ("gguf:q6_k", 1000, 8192, 20),
                                       ("gguf:q4_1", 500, 4096, 100), ("gguf:q2_k", 4096, 14336, 512),
                                       ("gguf:iq2_s", 12288, 1024, 200), ("gguf:q6_k", 4096, 14336, 384),
                                       ("gguf:q8_0", 1024, 4096, 1100)])
def test_gemm_split_k(fmt, N, K, M):
    """Shapes with few tiles and long K split K over workgroups (a workspace
    is given): split and unsplit products both meet the criterion on sampled
    rows, and each repeats bit for bit.  The last three have five eighths to
    two 64-row tiles per compute unit on 256 compute units (256, 384 and 192):
    K split in 4-span steps (with the weight rewritten once too above 256
    activation rows); [1024, 4096] x 1100 has 144 tiles: 3 splits in 8-span
    steps, the count rounded down to stay within 512 workgroups."""
    st, ws_bytes = nq.gemm_q8_1_workspace(fmt, N, K, M)
    assert st == 0 and ws_bytes > 0
    w = _weights(fmt, N, K, 55)
    _, xq = oracle.quantize_q8_1(_act(M, K, 56).astype(np.float32))
    announce(f"gemm split {fmt} [{N}, {K}] x {M}")
    a = _gemm(fmt, w, N, K, xq, split=True)
    b = _gemm(fmt, w, N, K, xq, split=False)
    a2 = _gemm(fmt, w, N, K, xq, split=True)
    b2 = _gemm(fmt, w, N, K, xq, split=False)
    assert np.array_equal(a.view(np.uint32), a2.view(np.uint32))
    assert np.array_equal(b.view(np.uint32), b2.view(np.uint32))
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, size=30)])
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(a[:, rows], ref, env, K, f"{fmt} split")
    linear_check(b[:, rows], ref, env, K, f"{fmt} unsplit")


def test_gemm_more_activation_rows_than_one_launch_takes():
    """65600 activation rows: the matrix-core product launches 65536 rows at a
    time; sampled activation rows on both sides of the boundary, every weight
    row, against the oracle."""
    fmt, N, K, M = "gguf:q8_0", 40, 64, 65600
    w = _weights(fmt, N, K, 91)
    x = _act(M, K, 92).astype(np.float32)
    _, xq = oracle.quantize_q8_1(x)
    announce(f"gemm {fmt} [{N}, {K}] x {M}")
    y = _gemm(fmt, w, N, K, xq)
    rows = np.r_[0:40, 65500:65600]
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, np.ascontiguousarray(xq[rows]), rows.size)
    linear_check(y[rows], ref, env, K, f"{fmt} M={M}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("N,K", [(300, 1024), (6144, 1024), (300, 1056)])
@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q2_k", "gguf:iq2_s", "gguf:q8_0", "gguf:tq1_0", "gguf:q5_1"])
def test_gemm_weight_rewritten_once_is_the_same_product(fmt, N, K):
    """Above 256 activation rows the weight is rewritten once per call into
    the workspace; the tiles then copy the same codes and scales they would
    rewrite themselves, so the bits equal the workspace-free product's (K below
    8 steps: no K split; 6144 weight rows make 864 tiles: 128-value K steps
    on 256 compute units, either way).  The rewrite stores a workgroup's
    scales through LDS when its 32 rows do not pass the last row (300 rows:
    the last workgroups do); K = 1056 (33 spans, 32-value formats only)
    leaves the last span octet short.  All rows (300) or sampled rows (6144)
    against the oracle."""
    if K % oracle.info(fmt)[1]:
        pytest.skip("K is not a whole number of this format's blocks")
    M = 1100
    st, ws_bytes = nq.gemm_q8_1_workspace(fmt, N, K, M)
    assert st == 0 and ws_bytes >= N * K
    w = _weights(fmt, N, K, 61)
    _, xq = oracle.quantize_q8_1(_act(M, K, 62).astype(np.float32))
    announce(f"gemm rewrite once {fmt} N={N}")
    a = _gemm(fmt, w, N, K, xq, w_off=1, split=True)
    b = _gemm(fmt, w, N, K, xq, w_off=1, split=False)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = np.arange(N) if N <= 300 else np.unique(np.r_[0, 127, 128, N - 1,
                                                         np.random.default_rng(N).integers(0, N, size=28)])
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(a[:, rows], ref, env, K, f"{fmt} N={N}")


@pytest.mark.parametrize("M", [3, 70])
def test_products_over_non_finite_scales(M):
    """A weight block with an infinite and one with a NaN binary16 scale: the
    outputs of those rows are non-finite in both the kernels and the oracle
    (which non-finite value may differ: the integer paths scale an exact
    integer sum); every other output meets the criterion."""
    fmt, N, K = "gguf:q8_0", 40, 256
    w = _weights(fmt, N, K, 71).copy()
    blk = w.reshape(N, K // 32, 34)
    blk[3, 1, 0:2] = [0x00, 0x7C]   # +inf
    blk[5, 0, 0:2] = [0x00, 0x7E]   # NaN
    _, xq = oracle.quantize_q8_1(_act(M, K, 72).astype(np.float32))
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    announce(f"non-finite scales M={M}")
    y = _gemm(fmt, w, N, K, xq)
    bad = np.zeros(N, bool)
    bad[[3, 5]] = True
    assert not np.any(np.isfinite(y[:, bad])) and not np.any(np.isfinite(ref[:, bad]))
    linear_check(y[:, ~bad], ref[:, ~bad], env[:, ~bad], K, f"{fmt} finite rows")


@pytest.mark.parametrize("fmt,N,K,M", [("gguf:q8_0", 1, 32, 5), ("gguf:q8_0", 1, 32, 33), ("gguf:q4_k", 1, 256, 32),
                                       ("gguf:q2_k", 3, 256, 65), ("gguf:iq1_m", 2, 256, 6), ("gguf:q6_k", 5, 256, 4)])
def test_gemm_tiny_shapes(fmt, N, K, M):
    """One weight row, one span or one block of K, activation rows at the
    boundaries of the tile heights and of the single-row kernel."""
    w = _weights(fmt, N, K, N + K + M)
    _, xq = oracle.quantize_q8_1(_act(M, K, 11).astype(np.float32))
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    announce(f"gemm tiny {fmt} [{N}, {K}] x {M}")
    for split in (True, False):
        y = _gemm(fmt, w, N, K, xq, w_off=1, split=split)
        linear_check(y, ref, env, K, f"{fmt} [{N}, {K}] x {M}")


@pytest.mark.parametrize("fmt,M", [("gguf:q4_k", 20), ("gguf:q8_0", 9), ("gguf:iq3_s", 40)])
def test_gemm_long_rows(fmt, M):
    """K = 28672 (112 K steps): many steps per workgroup, K split over
    workgroups, small-batch tile heights; sampled rows against the oracle."""
    N, K = 600, 28672
    w = _weights(fmt, N, K, 81)
    _, xq = oracle.quantize_q8_1(_act(M, K, 82).astype(np.float32))
    announce(f"gemm long rows {fmt} [{N}, {K}] x {M}")
    y = _gemm(fmt, w, N, K, xq)
    rows = np.unique(np.r_[0, 127, 128, N - 1, np.random.default_rng(M).integers(0, N, size=20)])
    sub = w.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq, M)
    linear_check(y[:, rows], ref, env, K, f"{fmt} K={K} M={M}")
