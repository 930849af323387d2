"""The C ABI on the host: exports, registry, length rule, error paths (no GPU).

Only entry points that return before touching the device are called here:
registry queries, nq_validate, and nq_dequantize_packed calls that fail
validation or have no elements.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import block_quantized_weight_nq_amd as nq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nq_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert set(declared) == set(nq.EXPORTS)
    lib = nq.library()
    for name in declared:
        assert hasattr(lib, name), name


def test_registry_matches_oracle_geometry():
    assert nq.format_count() == 28
    assert nq.format_names() == oracle.format_names()
    for i in range(nq.format_count()):
        info = nq.format_by_id(i)
        _, B, S, T = oracle.info(info.name.decode())
        assert (info.block_values, info.block_bytes, info.trailer_bytes) == (B, S, T)
        assert nq.format_query(info.name.decode()).id == i


@pytest.mark.parametrize("bad", ["GGUF:q4_0", "gguf:Q4_0", "q4_0", "gguf:q4_0(32)", "gguf:q4_0 ", "nvfp4:1",
                                 "gguf:", "", "gguf:nvfp4x", "NVFP4"])
def test_unknown_spellings_rejected(bad):
    info = nq.FormatInfo()
    assert nq.library().nq_format_query(bad.encode(), ctypes.byref(info)) == 2


def test_null_arguments():
    L = nq.library()
    assert L.nq_format_query(None, ctypes.byref(nq.FormatInfo())) == 1
    assert L.nq_format_query(b"gguf:q4_0", None) == 1
    assert L.nq_format_by_id(0, None) == 1
    assert L.nq_format_by_id(28, ctypes.byref(nq.FormatInfo())) == 2
    assert L.nq_format_by_id(-1, ctypes.byref(nq.FormatInfo())) == 2


SHAPES = [[256], [3, 512], [2, 3, 1024], [0, 256], [5, 0], [0], [4096, 14336], [7, 1, 256],
          [4, 31], [31], [0, 33], [-1, 256], [], [2 ** 40, 2 ** 40, 256], [2 ** 62, 0, 256], [1, 2 ** 61]]


@pytest.mark.parametrize("fmt", oracle.format_names())
def test_length_rule_agrees_with_oracle(fmt):
    ostatus = {oracle.OK: 0, oracle.ERR_RANK: 3, oracle.ERR_DIM: 4, oracle.ERR_ALIGN: 5, oracle.ERR_OVERFLOW: 7}
    for shape in SHAPES:
        st, nbytes, nelems = oracle.sizes(fmt, shape)
        want = ostatus[st]
        got, ne, _ = nq.validate_status(fmt, nbytes if st == oracle.OK else 0, shape, "f32")
        assert got == want, (fmt, shape, got, want)
        if st == oracle.OK:
            assert ne == nelems
            for delta in (-1, 1):
                if nbytes + delta >= 0:
                    assert nq.validate_status(fmt, nbytes + delta, shape)[0] == 6


def test_validate_reports_output_bytes():
    for code, size in (("f32", 4), ("f16", 2), ("bf16", 2), ("f64", 8)):
        ne, nb = nq.validate("gguf:q4_k", 144 * 6, [3, 512], code)
        assert (ne, nb) == (1536, 1536 * size)
    assert nq.validate_status("gguf:q4_k", 144 * 6, [3, 512], 4)[0] == 8
    assert nq.validate_status("gguf:q4_k", 144 * 6, [3, 512], -1)[0] == 8


def test_dequantize_rejects_bad_metadata_without_device():
    fid = nq.format_query("gguf:q8_0").id
    buf = np.zeros(64, dtype=np.uint8)
    p = buf.ctypes.data
    assert nq.dequantize_packed_raw(fid, p, 33, [32], 0, p, 0) == 6
    assert nq.dequantize_packed_raw(fid, p, 34, [31], 0, p, 0) == 5
    assert nq.dequantize_packed_raw(fid, p, 34, [32], 7, p, 0) == 8
    assert nq.dequantize_packed_raw(fid, 0, 34, [32], 0, p, 0) == 1
    assert nq.dequantize_packed_raw(fid, p, 34, [32], 0, 0, 0) == 1
    assert nq.dequantize_packed_raw(99, p, 34, [32], 0, p, 0) == 2
    # an element-misaligned output is refused before launch
    assert nq.dequantize_packed_raw(fid, p, 34, [32], 0, p + 2, 0) == 11
    # empty tensors succeed without launching (null pointers allowed)
    assert nq.dequantize_packed_raw(fid, 0, 0, [0, 32], 0, 0, 0) == 0
    nv = nq.format_query("nvfp4").id
    assert nq.dequantize_packed_raw(nv, p, 4, [0, 64], 2, 0, 0) == 0
    assert nq.dequantize_packed_raw(nv, p, 0, [0, 64], 2, 0, 0) == 6


def test_status_strings():
    for st in range(11):
        assert nq.library().nq_status_string(st) != b"unknown status"
    assert nq.library().nq_status_string(12345) == b"unknown status"


STACKED_CASES = [([12, 128], 1), ([12, 128], 2), ([12, 128], 3), ([12, 128], 4), ([12, 128], 5), ([12, 128], 12),
                 ([12, 128], 0), ([12, 128], -2), ([6, 0], 3), ([6, 0], 4), ([0, 128], 7), ([128], 1), ([128], 2),
                 ([12, 100], 2), ([3, 4, 64], 4), ([3, 4, 64], 8), ([12, 128], 1 << 30), ([12, 128], (1 << 30) + 1),
                 ([2 ** 40, 2 ** 40, 0], 1), ([-1, 64], 1), ([], 1)]


@pytest.mark.parametrize("shape,divisors", STACKED_CASES)
def test_nvfp4_stacked_length_rule_agrees_with_oracle(shape, divisors):
    ostatus = {oracle.OK: 0, oracle.ERR_RANK: 3, oracle.ERR_DIM: 4, oracle.ERR_ALIGN: 5, oracle.ERR_OVERFLOW: 7,
               oracle.ERR_DIVISORS: 10}
    st, nbytes, nelems = oracle.sizes_nvfp4_stacked(shape, divisors)
    want = ostatus[st]
    if want == 0 and divisors > (1 << 30):
        want = 10  # the library's own limit on the number of divisors
    got, ne, ob = nq.validate_nvfp4_stacked_status(nbytes if st == oracle.OK else 0, shape, divisors, "bf16")
    assert got == want, (shape, divisors, got, want)
    if got == 0:
        assert ne == nelems and ob == 2 * nelems
        for delta in (-4, -1, 1, 4):
            if nbytes + delta >= 0:
                assert nq.validate_nvfp4_stacked_status(nbytes + delta, shape, divisors)[0] == 6


def test_nvfp4_stacked_one_divisor_matches_plain_nvfp4_rule():
    for shape in ([12, 128], [0, 64], [3, 4, 64], [64]):
        st, nbytes, ne = oracle.sizes("nvfp4", shape)
        assert nq.validate_nvfp4_stacked_status(nbytes, shape, 1)[:2] == (0, ne)
        assert nq.validate_status("nvfp4", nbytes, shape)[:2] == (0, ne)


def test_nvfp4_stacked_rejects_before_device():
    buf = np.zeros(1024, dtype=np.uint8)
    p = buf.ctypes.data
    assert nq.dequantize_nvfp4_stacked_raw(p, 12 * 2 * 36 + 8, [12, 128], 3, 2, p, 0) == 6
    assert nq.dequantize_nvfp4_stacked_raw(p, 12 * 2 * 36 + 20, [12, 128], 5, 2, p, 0) == 10
    assert nq.dequantize_nvfp4_stacked_raw(p, 12 * 2 * 36 + 8, [12, 128], 2, 7, p, 0) == 8
    assert nq.dequantize_nvfp4_stacked_raw(0, 12 * 2 * 36 + 8, [12, 128], 2, 2, p, 0) == 1
    assert nq.dequantize_nvfp4_stacked_raw(p, 12 * 2 * 36 + 8, [12, 128], 2, 2, 0, 0) == 1
    assert nq.dequantize_nvfp4_stacked_raw(p, 12 * 2 * 36 + 8, [12, 128], 2, 2, p + 1, 0) == 11   # bf16 output misaligned
    # empty planes succeed without launching (null pointers allowed when nothing is read or written)
    assert nq.dequantize_nvfp4_stacked_raw(p, 12, [6, 0], 3, 2, 0, 0) == 0
    assert nq.dequantize_nvfp4_stacked_raw(0, 0, [6, 0], 3, 2, 0, 0) == 6


FP8_SHAPES = [[3, 5], [1, 1], [0, 5], [3, 0], [-1, 5], [15], [1, 3, 5], [], [2 ** 62, 4], [2 ** 31, 2 ** 31],
              [14336, 4096]]


@pytest.mark.parametrize("fmt", ["fp8_e4m3fn_row_bf16", "fp8_e4m3fn_row_fp16"])
@pytest.mark.parametrize("shape", FP8_SHAPES)
def test_fp8_row_length_rule_agrees_with_oracle(fmt, shape):
    ostatus = {oracle.OK: 0, oracle.ERR_RANK: 3, oracle.ERR_DIM: 4, oracle.ERR_OVERFLOW: 7}
    st, nbytes, nelems = oracle.sizes_fp8_row(shape)
    got, ne, ob = nq.validate_fp8_row_status(fmt, nbytes if st == oracle.OK else 0, shape, "f16")
    assert got == ostatus[st], (shape, got, st)
    if got == 0:
        assert ne == nelems and ob == 2 * nelems
        for delta in (-1, 1, -2, 2):
            assert nq.validate_fp8_row_status(fmt, nbytes + delta, shape)[0] == 6


def test_fp8_row_rejects_before_device():
    buf = np.zeros(64, dtype=np.uint8)
    p = buf.ctypes.data
    assert nq.validate_fp8_row_status(2, 21, [3, 5])[0] == 2      # unknown scale kind
    assert nq.validate_fp8_row_status(-1, 21, [3, 5])[0] == 2
    assert nq.validate_fp8_row_status(0, 21, [3, 5], 9)[0] == 8   # bad dtype
    assert nq.dequantize_fp8_row_raw(0, p, 20, [3, 5], 0, p, 0) == 6
    assert nq.dequantize_fp8_row_raw(0, 0, 21, [3, 5], 0, p, 0) == 1
    assert nq.dequantize_fp8_row_raw(0, p, 21, [3, 5], 0, 0, 0) == 1
    assert nq.dequantize_fp8_row_raw(0, p, 21, [3, 5], 0, p + 2, 0) == 11   # f32 output not element-aligned
    assert nq.dequantize_fp8_row_raw(1, p, 21, [15], 0, p, 0) == 3
    assert nq.dequantize_fp8_row_raw(1, p, 0, [0, 5], 0, p, 0) == 4


@pytest.mark.parametrize("scheme,G", [("q4_g64_fp16", 64), ("q8_g32_fp16", 32)])
def test_grouped_absmax_validation(scheme, G):
    assert nq.validate_grouped_absmax_status(scheme, [3, 70]) == (0, 210, 3 * ((70 + G - 1) // G) * 2)
    assert nq.validate_grouped_absmax_status(scheme, [3, 70], "bf16")[0] == 0
    assert nq.validate_grouped_absmax_status(scheme, [3, 70], 7)[0] == 8
    assert nq.validate_grouped_absmax_status(scheme, [210])[0] == 3
    assert nq.validate_grouped_absmax_status(scheme, [0, 70])[0] == 4
    assert nq.validate_grouped_absmax_status(scheme, [3, -1])[0] == 4
    assert nq.validate_grouped_absmax_status(scheme, [1, 1 << 31])[0] == 7
    assert nq.validate_grouped_absmax_status(scheme, [1 << 40, 1 << 30])[0] == 7
    assert nq.validate_grouped_absmax_status(9, [3, 70])[0] == 2


def test_grouped_absmax_rejects_before_device():
    buf = np.zeros(64, dtype=np.uint32)
    p = buf.ctypes.data
    assert nq.quantize_grouped_absmax_raw(0, 0, [2, 8], 0, p, p, p, 0) == 1
    assert nq.quantize_grouped_absmax_raw(0, p, [2, 8], 0, p, p, 0, 0) == 1
    assert nq.quantize_grouped_absmax_raw(0, p + 2, [2, 8], 0, p, p, p, 0) == 11   # f32 source misaligned
    assert nq.quantize_grouped_absmax_raw(0, p, [2, 8], 0, p, p + 1, p, 0) == 11   # scales misaligned
    assert nq.quantize_grouped_absmax_raw(0, p, [2, 8], 0, p, p, p + 2, 0) == 11   # status misaligned
    assert nq.quantize_grouped_absmax_raw(4, p, [2, 8], 0, p, p, p, 0) == 2


def test_quantize_q8_1_validation():
    assert nq.validate_quantize_q8_1_status([3, 64]) == (0, 3 * 2 * 36)
    assert nq.validate_quantize_q8_1_status([1, 4096], "bf16") == (0, 128 * 36)
    assert nq.validate_quantize_q8_1_status([3, 64], 7)[0] == 8
    assert nq.validate_quantize_q8_1_status([192])[0] == 3
    assert nq.validate_quantize_q8_1_status([0, 64])[0] == 4
    assert nq.validate_quantize_q8_1_status([3, -32])[0] == 4
    assert nq.validate_quantize_q8_1_status([3, 48])[0] == 5
    assert nq.validate_quantize_q8_1_status([1 << 40, 1 << 30])[0] == 7


def test_quantize_q8_1_rejects_before_device():
    buf = np.zeros(64, dtype=np.uint32)
    p = buf.ctypes.data
    assert nq.quantize_q8_1_raw(0, [2, 32], 0, p, p, 0) == 1
    assert nq.quantize_q8_1_raw(p, [2, 32], 0, 0, p, 0) == 1
    assert nq.quantize_q8_1_raw(p, [2, 32], 0, p, 0, 0) == 1
    assert nq.quantize_q8_1_raw(p + 2, [2, 32], 0, p, p, 0) == 11   # f32 source misaligned
    assert nq.quantize_q8_1_raw(p, [2, 32], 0, p + 2, p, 0) == 11   # blocks misaligned
    assert nq.quantize_q8_1_raw(p, [2, 32], 0, p, p + 1, 0) == 11   # status misaligned
    assert nq.quantize_q8_1_raw(p, [2, 33], 0, p, p, 0) == 5
    assert nq.quantize_q8_1_raw(p, [2, 32], 9, p, p, 0) == 8


@pytest.mark.parametrize("fmt", [f for f in oracle.format_names() if f.startswith("gguf:")])
def test_gemv_length_rule_agrees_with_oracle(fmt):
    _, B, S, _ = oracle.info(fmt)
    N, K = 3, 2 * B
    assert nq.validate_gemv_q8_1_status(fmt, N * 2 * S, N, K, 1) == 0
    assert nq.validate_gemv_q8_1_status(fmt, N * 2 * S, N, K, 8) == 0
    assert nq.validate_gemv_q8_1_status(fmt, N * 2 * S + 1, N, K, 1) == 6
    assert nq.validate_gemv_q8_1_status(fmt, N * 2 * S, N, K, 9) == 4
    assert nq.validate_gemv_q8_1_status(fmt, N * 2 * S, N, K, 0) == 4
    assert nq.validate_gemv_q8_1_status(fmt, 0, 0, K, 1) == 4
    assert nq.validate_gemv_q8_1_status(fmt, N * 2 * S, N, K + 32 if B > 32 else K + 16, 1) == 5
    assert oracle.sizes(fmt, [N, K])[1] == N * 2 * S


def test_gemv_rejects_before_device():
    buf = np.zeros(256, dtype=np.uint32)
    p = buf.ctypes.data
    q8 = nq.format_query("gguf:q8_0").id
    assert nq.validate_gemv_q8_1_status("nvfp4", 40, 1, 64, 1) == 2
    assert nq.validate_gemv_q8_1_status(99, 34, 1, 32, 1) == 2
    assert nq.validate_gemv_q8_1_status(q8, 34 << 31, 1 << 31, 32, 1) == 7
    assert nq.gemv_q8_1_raw(q8, 0, 34, 1, 32, p, 1, p, 0) == 1
    assert nq.gemv_q8_1_raw(q8, p, 34, 1, 32, 0, 1, p, 0) == 1
    assert nq.gemv_q8_1_raw(q8, p, 34, 1, 32, p, 1, 0, 0) == 1
    assert nq.gemv_q8_1_raw(q8, p, 34, 1, 32, p + 2, 1, p, 0) == 11   # activation blocks misaligned
    assert nq.gemv_q8_1_raw(q8, p, 34, 1, 32, p, 1, p + 2, 0) == 11   # output misaligned
    assert nq.gemv_q8_1_raw(q8, p, 35, 1, 32, p, 1, p, 0) == 6


@pytest.mark.parametrize("fmt", ["gguf:q8_0", "gguf:q4_k", "gguf:iq2_xxs", "gguf:tq1_0", "gguf:nvfp4"])
def test_gemm_validation(fmt):
    """The batched product takes any M >= 1 and otherwise checks as the
    single-row product."""
    _, B, S, _ = oracle.info(fmt)
    N, K = 3, 2 * B
    for M in (1, 8, 9, 64, 5000):
        assert nq.validate_gemm_q8_1_status(fmt, N * 2 * S, N, K, M) == 0
    assert nq.validate_gemm_q8_1_status(fmt, N * 2 * S, N, K, 0) == 4
    assert nq.validate_gemm_q8_1_status(fmt, N * 2 * S, N, K, -1) == 4
    assert nq.validate_gemm_q8_1_status(fmt, N * 2 * S + 1, N, K, 9) == 6
    assert nq.validate_gemm_q8_1_status(fmt, 0, 0, K, 9) == 4
    assert nq.validate_gemm_q8_1_status(fmt, N * 2 * S, N, K + 32 if B > 32 else K + 16, 9) == 5
    assert nq.validate_gemm_q8_1_status(fmt, N * 2 * S, N, K, 1 << 31) == 7


def test_gemm_rejects_before_device():
    buf = np.zeros(256, dtype=np.uint32)
    p = buf.ctypes.data
    q8 = nq.format_query("gguf:q8_0").id
    assert nq.validate_gemm_q8_1_status("nvfp4", 40, 1, 64, 9) == 2
    assert nq.validate_gemm_q8_1_status(99, 34, 1, 32, 9) == 2
    assert nq.validate_gemm_q8_1_status(q8, 34 << 31, 1 << 31, 32, 9) == 7
    # output bytes M * N * 4 past 2^63 - 1, then just below
    assert nq.validate_gemm_q8_1_status(q8, 34 * ((1 << 31) - 1), (1 << 31) - 1, 32, (1 << 31) - 1) == 7
    assert nq.validate_gemm_q8_1_status(q8, 34 * ((1 << 31) - 1), (1 << 31) - 1, 32, 1 << 30) == 0
    assert nq.gemm_q8_1_raw(q8, 0, 34, 1, 32, p, 9, p, 0, 0, 0) == 1
    assert nq.gemm_q8_1_raw(q8, p, 34, 1, 32, 0, 9, p, 0, 0, 0) == 1
    assert nq.gemm_q8_1_raw(q8, p, 34, 1, 32, p, 9, 0, 0, 0, 0) == 1
    assert nq.gemm_q8_1_raw(q8, p, 34, 1, 32, p + 2, 9, p, 0, 0, 0) == 11   # activation blocks misaligned
    assert nq.gemm_q8_1_raw(q8, p, 34, 1, 32, p, 9, p + 2, 0, 0, 0) == 11   # output misaligned
    assert nq.gemm_q8_1_raw(q8, p, 35, 1, 32, p, 9, p, 0, 0, 0) == 6
    assert nq.gemm_q8_1_raw(q8, p, 34, 1, 32, p, 9, p, p + 8, 64, 0) == 11   # workspace not 16-byte aligned


def test_gemm_workspace_sizes():
    """The workspace holds the K-split partials (5 rows or more, few tiles,
    long K; no GPU: 256 compute units assumed) and, above 256 activation rows,
    the weight rewritten once: N K code bytes, then K / 32 * NH * N binary32
    scales and, for the affine formats, as many offsets (each part rounded
    up to 256 bytes)."""
    assert nq.gemm_q8_1_workspace("gguf:q4_k", 4096, 14336, 4) == (0, 0)          # single-row kernel
    assert nq.gemm_q8_1_workspace("gguf:q4_k", 4096, 14336, 5)[1] > 0            # matrix cores, K split
    assert nq.gemm_q8_1_workspace("gguf:q4_k", 4096, 1024, 64) == (0, 0)      # 4 K steps, one activation tile
    st, b = nq.gemm_q8_1_workspace("gguf:q4_k", 4096, 14336, 64)              # 32 tiles, 56 steps: split only
    assert st == 0 and b > 0 and b % (64 * 4096 * 4) == 0
    assert 2 <= b // (64 * 4096 * 4) <= 14
    assert nq.gemm_q8_1_workspace("gguf:tq1_0", 4096, 14336, 64)[1] > 0
    # 3584 tiles: no split; q4_k: 14336 * 4096 code bytes, scales and offsets 128 * 14336 * 4 each
    assert nq.gemm_q8_1_workspace("gguf:q4_k", 14336, 4096, 2048) == (0, 58720256 + 2 * 7340032)
    # q6_k: two scales per span, no offsets
    assert nq.gemm_q8_1_workspace("gguf:q6_k", 14336, 4096, 2048) == (0, 58720256 + 2 * 7340032)
    assert nq.gemm_q8_1_workspace("gguf:q8_0", 14336, 4096, 2048) == (0, 58720256 + 7340032)
    # 256 tiles, one per compute unit: three K splits (3 * 512 * 4096 binary32), then the rewrite
    # (4096 * 14336 code bytes, 448 * 4096 scales)
    assert nq.gemm_q8_1_workspace("gguf:q8_0", 4096, 14336, 512) == (0, 25165824 + 58720256 + 7340032)
    # 448 tiles (under two per compute unit): two K splits in 4-span steps (2 * 256 * 14336 binary32)
    assert nq.gemm_q8_1_workspace("gguf:q8_0", 14336, 1024, 256) == (0, 29360128)
    # 1024 and 1280 tiles: no split; the rewrite from 257 rows (32768 * 1024 code bytes, 32 * 32768 scales)
    assert nq.gemm_q8_1_workspace("gguf:q8_0", 32768, 1024, 256) == (0, 0)
    assert nq.gemm_q8_1_workspace("gguf:q8_0", 32768, 1024, 257) == (0, 33554432 + 4194304)
    assert nq.gemm_q8_1_workspace("nvfp4", 1, 64, 9)[0] == 2
    assert nq.gemm_q8_1_workspace("gguf:q4_k", 1, 100, 9)[0] == 5


def test_status_strings_name_every_status():
    L = nq.library()
    for st, name in nq.STATUS_NAMES.items():
        text = L.nq_status_string(st).decode()
        assert text and text != "unknown status", (st, name)
    assert L.nq_status_string(13).decode() == "unknown status"
    assert "NULL" in L.nq_status_string(1).decode() and "align" in L.nq_status_string(11).decode()


def test_many_tensor_decode_rejects_before_device():
    """nq_dequantize_packed_many validates every tensor first and names the
    first failing one; none of these calls reaches a launch."""
    buf = np.zeros(256, dtype=np.uint32)
    p = buf.ctypes.data
    q4k, q8, nv = (nq.format_query(f).id for f in ("gguf:q4_k", "gguf:q8_0", "nvfp4"))
    L = nq.library()
    failed = ctypes.c_int32(5)
    assert L.nq_dequantize_packed_many(None, 0, 2, ctypes.byref(failed), None) == 0 and failed.value == -1
    assert L.nq_dequantize_packed_many(None, -1, 2, ctypes.byref(failed), None) == 4
    assert L.nq_dequantize_packed_many(None, 3, 2, ctypes.byref(failed), None) == 1
    assert L.nq_dequantize_packed_many(None, 1, 2, None, None) == 1
    assert nq.dequantize_packed_many_raw([], 2, 0) == (0, -1)
    ok = (q4k, p, 144, [256], p)
    assert nq.dequantize_packed_many_raw([ok], 4, 0) == (8, -1)                         # bad dtype
    assert nq.dequantize_packed_many_raw([ok, (q4k, p, 145, [256], p)], 2, 0) == (6, 1)  # length rule
    assert nq.dequantize_packed_many_raw([ok, ok, (99, p, 34, [32], p)], 2, 0) == (2, 2)
    assert nq.dequantize_packed_many_raw([ok, (q8, p, 34, [31], p)], 2, 0) == (5, 1)
    assert nq.dequantize_packed_many_raw([(q8, p, 34, [-1, 32], p)], 2, 0) == (4, 0)
    assert nq.dequantize_packed_many_raw([(q8, 0, 34, [32], p)], 2, 0) == (1, 0)        # NULL payload
    assert nq.dequantize_packed_many_raw([(q8, p, 34, [32], 0)], 2, 0) == (1, 0)        # NULL out
    assert nq.dequantize_packed_many_raw([(q8, p, 34, [32], p + 1)], 2, 0) == (11, 0)   # bf16 out misaligned
    assert nq.dequantize_packed_many_raw([(q8, p, 34, [32], p + 2)], 0, 0) == (11, 0)   # f32 out misaligned
    assert nq.dequantize_packed_many_raw([(nv, p, 40, [64], p + 4)], 3, 0) == (11, 0)  # f64 out misaligned
    # empty tensors need no pointers; a failure after them is still reported by index
    empty = (q4k, 0, 0, [0, 256], 0)
    assert nq.dequantize_packed_many_raw([empty, empty, (nv, p, 4, [0, 64], 0), (nv, p, 3, [0, 64], 0)], 2, 0) \
        == (6, 3)
    assert nq.dequantize_packed_many_raw([empty, (nv, 0, 4, [5, 0], 0)], 2, 0) == (1, 1)   # trailer: payload needed


def test_measure_stream_rejects_before_device():
    buf = np.zeros(256, dtype=np.uint32)
    p = (buf.ctypes.data + 15) // 16 * 16
    assert nq.measure_stream_raw(0, 32, p, 32, 1, 0, 0) == 1
    assert nq.measure_stream_raw(p, 32, 0, 32, 1, 0, 0) == 1
    assert nq.measure_stream_raw(p + 8, 32, p, 32, 1, 0, 0) == 11
    assert nq.measure_stream_raw(p, 32, p + 4, 32, 1, 0, 0) == 11
    assert nq.measure_stream_raw(p, 48, p, 32, 1, 0, 0) == 4       # reads more than it writes
    assert nq.measure_stream_raw(p, 8, p, 32, 1, 0, 0) == 4        # not a multiple of 16
    assert nq.measure_stream_raw(p, 0, p, 0, 1, 0, 0) == 4
    for c in (0, 3, 16, -1):
        assert nq.measure_stream_raw(p, 16, p, 32, c, 0, 0) == 4   # chunks per thread not 1, 2, 4, 8
    assert nq.measure_stream_raw(p, 16, p, 32, 2, 4, 0) == 4       # unknown flag bit
    assert nq.measure_stream_raw(p, 16, p, (1 << 40) + 16, 1, 0, 0) == 7


def test_gemm_noalloc_refuses_shapes_past_its_scratch_before_device():
    """The no-allocation product checks as nq_gemm_q8_1 and refuses a shape
    whose workspace passes its 32 MiB scratch (NQ_ERR_SCRATCH) before any
    device work."""
    buf = np.zeros(64, dtype=np.uint32)
    p = buf.ctypes.data
    q4k = nq.format_query("gguf:q4_k").id
    nb = 14336 * 4096 // 256 * 144
    st, need = nq.gemm_q8_1_workspace("gguf:q4_k", 14336, 4096, 512)
    assert st == 0 and need > nq.GEMM_SCRATCH_BYTES
    assert nq.gemm_q8_1_noalloc_raw(q4k, p, nb, 14336, 4096, p, 512, p, 0) == 12
    assert nq.gemm_q8_1_noalloc_raw(q4k, p, nb + 1, 14336, 4096, p, 512, p, 0) == 6
    assert nq.gemm_q8_1_noalloc_raw(nq.format_query("nvfp4").id, p, 40, 1, 64, p, 9, p, 0) == 2
    assert nq.gemm_q8_1_noalloc_raw(q4k, p, nb, 14336, 4096, p, 0, p, 0) == 4
    assert nq.gemm_q8_1_noalloc_raw(q4k, 0, nb, 14336, 4096, p, 64, p, 0) == 1
    assert nq.gemm_q8_1_noalloc_raw(q4k, p, nb, 14336, 4096, p + 2, 64, p, 0) == 11
