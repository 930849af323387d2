"""ctypes wrapper of the C oracle (``nq_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain, single-threaded CPU
definition of packed-weight decoding that the HIP library is checked
against.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package; the product library never does.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# NQ_SANITIZE=1: a separate build under AddressSanitizer and
# UndefinedBehaviorSanitizer (clang, whose runtime the sanitized test run
# preloads; see tests/run_sanitized.py)
SANITIZE = os.environ.get("NQ_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")
_SRC = os.path.join(_HERE, "nq_oracle.c")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

# -O1, no contraction, no fast-math: each float operation is one IEEE
# binary32 operation (x86-64 SSE), as the decoding rules require.
CFLAGS = ["-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
_NP_OUT = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}

OK, ERR_FORMAT, ERR_RANK, ERR_DIM, ERR_ALIGN, ERR_OVERFLOW, ERR_LENGTH, ERR_DTYPE, ERR_DIVISORS = range(9)

_lib = None


def build():
    """Compile liboracle.so with gcc (NQ_SANITIZE=1: liboracle_san.so with clang and the sanitizers)."""
    if SANITIZE:
        subprocess.run(["/opt/rocm/llvm/bin/clang", *CFLAGS, *SAN_FLAGS, "-o", _LIB_PATH, _SRC, "-lm"], check=True)
    else:
        subprocess.run(["gcc", *CFLAGS, "-o", _LIB_PATH, _SRC, "-lm"], check=True)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        c = ctypes
        L.nqo_format_count.restype = c.c_int
        L.nqo_format_info.argtypes = [c.c_int, c.POINTER(c.c_char_p), c.POINTER(c.c_int),
                                      c.POINTER(c.c_int), c.POINTER(c.c_int)]
        L.nqo_format_find.argtypes = [c.c_char_p]
        L.nqo_sizes.argtypes = [c.c_int, c.POINTER(c.c_int64), c.c_int, c.POINTER(c.c_uint64),
                                c.POINTER(c.c_uint64)]
        L.nqo_decode.argtypes = [c.c_int, c.c_void_p, c.c_uint64, c.POINTER(c.c_int64), c.c_int,
                                 c.c_int, c.c_void_p]
        L.nqo_decode_blocks_f32.argtypes = [c.c_int, c.c_void_p, c.c_uint64, c.c_float, c.c_void_p]
        L.nqo_sizes_fp8_row.argtypes = [c.POINTER(c.c_int64), c.c_int, c.POINTER(c.c_uint64), c.POINTER(c.c_uint64)]
        L.nqo_decode_fp8_row.argtypes = [c.c_int, c.c_void_p, c.c_uint64, c.POINTER(c.c_int64), c.c_int, c.c_int,
                                         c.c_void_p]
        L.nqo_bf16_to_f32.argtypes = [c.c_uint16]
        L.nqo_bf16_to_f32.restype = c.c_float
        L.nqo_grouped_absmax.argtypes = [c.c_int, c.c_int, c.c_void_p, c.c_int64, c.c_int64, c.c_void_p, c.c_void_p]
        L.nqo_sizes_nvfp4_stacked.argtypes = [c.POINTER(c.c_int64), c.c_int, c.c_int64, c.POINTER(c.c_uint64),
                                              c.POINTER(c.c_uint64)]
        L.nqo_decode_nvfp4_stacked.argtypes = [c.c_void_p, c.c_uint64, c.POINTER(c.c_int64), c.c_int, c.c_int64,
                                               c.c_int, c.c_void_p]
        L.nqo_f16_to_f32.argtypes = [c.c_uint16]
        L.nqo_f16_to_f32.restype = c.c_float
        L.nqo_f32_to_bf16.argtypes = [c.c_float]
        L.nqo_f32_to_bf16.restype = c.c_uint16
        L.nqo_f32_to_f16.argtypes = [c.c_float]
        L.nqo_f32_to_f16.restype = c.c_uint16
        L.nqo_e4m3fn_to_f32.argtypes = [c.c_uint8]
        L.nqo_e4m3fn_to_f32.restype = c.c_float
        L.nqo_convert.argtypes = [c.c_void_p, c.c_uint64, c.c_int, c.c_void_p]
        L.nqo_quantize_q8_1.argtypes = [c.c_int, c.c_void_p, c.c_int64, c.c_int64, c.c_void_p]
        L.nqo_gemv_q8_1.argtypes = [c.c_int, c.c_void_p, c.c_uint64, c.c_int64, c.c_int64, c.c_void_p, c.c_int64,
                                    c.c_void_p, c.c_void_p]
        L.nqo_grid_rows.argtypes = [c.c_int]
        L.nqo_grid_width.argtypes = [c.c_int]
        L.nqo_grid_value.argtypes = [c.c_int, c.c_int, c.c_int]
        _lib = L
    return _lib


def format_names():
    L = lib()
    out = []
    for i in range(L.nqo_format_count()):
        name = ctypes.c_char_p()
        L.nqo_format_info(i, ctypes.byref(name), None, None, None)
        out.append(name.value.decode())
    return out


def info(fmt):
    """(index, B, S, trailer) for a format name."""
    L = lib()
    idx = L.nqo_format_find(fmt.encode())
    if idx < 0:
        raise KeyError(fmt)
    B, S, T = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    L.nqo_format_info(idx, None, ctypes.byref(B), ctypes.byref(S), ctypes.byref(T))
    return idx, B.value, S.value, T.value


def _shape_arg(shape):
    arr = (ctypes.c_int64 * max(1, len(shape)))(*shape)
    return arr, len(shape)


def sizes(fmt, shape):
    """(status, nbytes, nelems) of the length rule for a format index or name."""
    idx = fmt if isinstance(fmt, int) else lib().nqo_format_find(fmt.encode())
    arr, rank = _shape_arg(shape)
    nb, ne = ctypes.c_uint64(), ctypes.c_uint64()
    st = lib().nqo_sizes(idx, arr, rank, ctypes.byref(nb), ctypes.byref(ne))
    return st, nb.value, ne.value


def decode(fmt, payload, shape, dtype="f32"):
    """Decode a whole payload; returns a flat array (raw 16-bit words for f16/bf16)."""
    idx = lib().nqo_format_find(fmt.encode())
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    st, nbytes, nelems = sizes(idx, shape)
    if st != OK:
        raise ValueError(f"oracle length rule rejects {fmt} {shape}: status {st}")
    out = np.empty(nelems, dtype=_NP_OUT[dtype])
    arr, rank = _shape_arg(shape)
    st = lib().nqo_decode(idx, payload.ctypes.data, payload.size, arr, rank, DTYPES[dtype],
                          out.ctypes.data)
    if st != OK:
        raise ValueError(f"oracle decode of {fmt} {shape} failed: status {st}")
    return out


def decode_status(fmt, payload, shape, dtype="f32"):
    """Status code only (for length-rule tests); decodes into scratch on success."""
    idx = lib().nqo_format_find(fmt.encode())
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    st, nbytes, nelems = sizes(idx, shape) if idx >= 0 else (ERR_FORMAT, 0, 0)
    out = np.empty(max(1, nelems if st == OK else 1), dtype=np.float64)
    arr, rank = _shape_arg(shape)
    return lib().nqo_decode(idx, payload.ctypes.data, payload.size, arr, rank,
                            DTYPES.get(dtype, 99), out.ctypes.data)


def sizes_nvfp4_stacked(shape, divisors):
    """(status, nbytes, nelems) of the stacked-divisor nvfp4 length rule."""
    arr, rank = _shape_arg(shape)
    nb, ne = ctypes.c_uint64(), ctypes.c_uint64()
    st = lib().nqo_sizes_nvfp4_stacked(arr, rank, divisors, ctypes.byref(nb), ctypes.byref(ne))
    return st, nb.value, ne.value


def decode_nvfp4_stacked(payload, shape, divisors, dtype="f32"):
    """Decode an nvfp4 plane of `divisors` stacked sources (flat array, raw 16-bit words for f16/bf16)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    st, nbytes, nelems = sizes_nvfp4_stacked(shape, divisors)
    if st != OK:
        raise ValueError(f"oracle length rule rejects nvfp4 {shape} divisors={divisors}: status {st}")
    out = np.empty(nelems, dtype=_NP_OUT[dtype])
    arr, rank = _shape_arg(shape)
    st = lib().nqo_decode_nvfp4_stacked(payload.ctypes.data, payload.size, arr, rank, divisors, DTYPES[dtype],
                                        out.ctypes.data)
    if st != OK:
        raise ValueError(f"oracle decode of nvfp4 {shape} divisors={divisors} failed: status {st}")
    return out


FP8_ROW_KINDS = {"fp8_e4m3fn_row_bf16": 0, "fp8_e4m3fn_row_fp16": 1}


def sizes_fp8_row(shape):
    """(status, nbytes, nelems) of the row-scaled FP8 length rule."""
    arr, rank = _shape_arg(shape)
    nb, ne = ctypes.c_uint64(), ctypes.c_uint64()
    st = lib().nqo_sizes_fp8_row(arr, rank, ctypes.byref(nb), ctypes.byref(ne))
    return st, nb.value, ne.value


def decode_fp8_row(fmt, payload, shape, dtype="f32"):
    """Decode a row-scaled FP8 matrix (flat array, raw 16-bit words for f16/bf16)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    st, nbytes, nelems = sizes_fp8_row(shape)
    if st != OK:
        raise ValueError(f"oracle length rule rejects {fmt} {shape}: status {st}")
    out = np.empty(nelems, dtype=_NP_OUT[dtype])
    arr, rank = _shape_arg(shape)
    st = lib().nqo_decode_fp8_row(FP8_ROW_KINDS[fmt], payload.ctypes.data, payload.size, arr, rank, DTYPES[dtype],
                                  out.ctypes.data)
    if st != OK:
        raise ValueError(f"oracle decode of {fmt} {shape} failed: status {st}")
    return out


GQ_SCHEMES = {"q4_g64_fp16": (0, 64, -8, 7), "q5_g64_fp16": (1, 64, -16, 15), "q6_g64_fp16": (2, 64, -32, 31),
              "q8_g32_fp16": (3, 32, -127, 127)}
_IN_DTYPES = {"f32": (0, np.float32), "f16": (1, np.uint16), "bf16": (2, np.uint16), "f64": (3, np.float64)}


def grouped_absmax(scheme, x, in_dtype="f32"):
    """grouped_absmax of a [N, K] array (f16/bf16 given as raw uint16 words).
    Returns (status, codes int8 [N, K], scales uint16 [N, ceil(K/G)])."""
    sid, G, _, _ = GQ_SCHEMES[scheme]
    code, npt = _IN_DTYPES[in_dtype]
    x = np.ascontiguousarray(x, dtype=npt)
    N, K = x.shape
    codes = np.zeros((N, K), dtype=np.int8)
    scales = np.zeros((N, (K + G - 1) // G), dtype=np.uint16)
    st = lib().nqo_grouped_absmax(sid, code, x.ctypes.data, N, K, codes.ctypes.data, scales.ctypes.data)
    if st < 0:
        raise ValueError(f"oracle grouped_absmax rejects {scheme} {x.shape} {in_dtype}")
    return st, codes, scales


def quantize_q8_1(x, in_dtype="f32"):
    """q8_1 activation blocks of a [M, K] array (K % 32 == 0; f16/bf16 given as
    raw uint16 words).  Returns (status, blocks uint8 [M, K/32, 36])."""
    code, npt = _IN_DTYPES[in_dtype]
    x = np.ascontiguousarray(x, dtype=npt)
    M, K = x.shape
    blocks = np.zeros((M, K // 32, 36), dtype=np.uint8)
    st = lib().nqo_quantize_q8_1(code, x.ctypes.data, M, K, blocks.ctypes.data)
    if st < 0:
        raise ValueError(f"oracle quantize_q8_1 rejects {x.shape} {in_dtype}")
    return st, blocks


def gemv_q8_1(fmt, weight, N, K, xq, M):
    """y[M, N] = x_hat[M, K] @ w_hat[N, K]^T in binary64 and the criterion's
    scale env[M, N] (see nqo_gemv_q8_1)."""
    idx = info(fmt)[0]
    weight = np.ascontiguousarray(weight, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.empty((M, N), dtype=np.float64)
    env = np.empty((M, N), dtype=np.float64)
    st = lib().nqo_gemv_q8_1(idx, weight.ctypes.data, weight.size, N, K, xq.ctypes.data, M, y.ctypes.data,
                             env.ctypes.data)
    if st != OK:
        raise ValueError(f"oracle gemv_q8_1 of {fmt} [{N}, {K}] x {M} failed: status {st}")
    return y, env


def bf16_to_f32(w):
    return lib().nqo_bf16_to_f32(w)


def decode_blocks_f32(fmt, blocks, d_w=0.0):
    """Decode back-to-back blocks (no trailer) to float32."""
    idx, B, S, _ = info(fmt)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    n = blocks.size // S
    out = np.empty(n * B, dtype=np.float32)
    lib().nqo_decode_blocks_f32(idx, blocks.ctypes.data, n, ctypes.c_float(d_w), out.ctypes.data)
    return out


def convert(x, dtype):
    """Convert a float32 array with the oracle's conversion to `dtype` (raw words)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=_NP_OUT[dtype])
    lib().nqo_convert(x.ctypes.data, x.size, DTYPES[dtype], out.ctypes.data)
    return out


def f16_to_f32(h):
    return lib().nqo_f16_to_f32(h)


def e4m3fn_to_f32(w):
    return lib().nqo_e4m3fn_to_f32(w)


BOOKS = ["iq2xxs_grid", "iq2xs_grid", "iq2s_grid", "iq3xxs_grid", "iq3s_grid", "iq1s_grid"]


def grid(book):
    """The expanded codebook as an int array [rows, width]."""
    k = BOOKS.index(book)
    L = lib()
    rows, width = L.nqo_grid_rows(k), L.nqo_grid_width(k)
    return np.array([[L.nqo_grid_value(k, r, j) for j in range(width)] for r in range(rows)],
                    dtype=np.int32)


def grid_bad_fields():
    return lib().nqo_grid_bad_fields()
