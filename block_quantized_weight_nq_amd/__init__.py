"""Python binding of libnq.so, the MI355X (gfx950) packed-weight decoder.

Argument marshalling only: every step of a decode runs in the library's HIP
kernels behind the C ABI of include/nq.h.  PyTorch supplies device memory
and streams.  There is no fallback: if libnq.so is missing, every call raises.

    import torch, block_quantized_weight_nq_amd as nq
    y = nq.dequantize_packed("gguf:q4_k", payload_u8_cuda, [4096, 4096], torch.bfloat16)
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnq.so")

NQ_OK = 0
STATUS_NAMES = {0: "NQ_OK", 1: "NQ_ERR_NULL_ARG", 2: "NQ_ERR_UNKNOWN_FORMAT", 3: "NQ_ERR_BAD_RANK",
                4: "NQ_ERR_BAD_DIM", 5: "NQ_ERR_NOT_BLOCK_ALIGNED", 6: "NQ_ERR_LENGTH_MISMATCH",
                7: "NQ_ERR_OVERFLOW", 8: "NQ_ERR_BAD_DTYPE", 9: "NQ_ERR_HIP", 10: "NQ_ERR_BAD_DIVISORS",
                11: "NQ_ERR_MISALIGNED", 12: "NQ_ERR_SCRATCH"}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
FAMILIES = {0: "simple", 1: "kquant", 2: "iq", 3: "fp4", 4: "ternary"}
EXPORTS = ["nq_format_count", "nq_format_by_id", "nq_format_query", "nq_validate",
           "nq_dequantize_packed", "nq_dequantize_packed_many", "nq_measure_stream", "nq_validate_nvfp4_stacked", "nq_dequantize_nvfp4_stacked",
           "nq_validate_fp8_row", "nq_dequantize_fp8_row", "nq_validate_grouped_absmax",
           "nq_quantize_grouped_absmax", "nq_validate_quantize_q8_1", "nq_quantize_q8_1",
           "nq_validate_gemv_q8_1", "nq_gemv_q8_1", "nq_validate_gemm_q8_1", "nq_gemm_q8_1_workspace", "nq_gemm_q8_1", "nq_gemm_q8_1_noalloc",
           "nq_status_string"]
GEMV_MAX_M = 8
GQ_SCHEMES = {"q4_g64_fp16": (0, 64), "q5_g64_fp16": (1, 64), "q6_g64_fp16": (2, 64), "q8_g32_fp16": (3, 32)}
FP8_ROW_KINDS = {"fp8_e4m3fn_row_bf16": 0, "fp8_e4m3fn_row_fp16": 1}


class NqError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        msg = _lib().nq_status_string(status).decode()
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}{(' (' + what + ')') if what else ''}")


class FormatInfo(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("name", ctypes.c_char_p), ("block_values", ctypes.c_int32),
                ("block_bytes", ctypes.c_int32), ("trailer_bytes", ctypes.c_int32),
                ("family", ctypes.c_int32)]

    def __repr__(self):
        return (f"FormatInfo(id={self.id}, name={self.name.decode()!r}, B={self.block_values}, "
                f"S={self.block_bytes}, trailer={self.trailer_bytes}, family={FAMILIES[self.family]})")


class TensorDesc(ctypes.Structure):
    """nq_tensor: one tensor of nq_dequantize_packed_many."""
    _fields_ = [("format", ctypes.c_int32), ("rank", ctypes.c_int32), ("shape", ctypes.POINTER(ctypes.c_int64)),
                ("payload", ctypes.c_void_p), ("nbytes", ctypes.c_uint64), ("out", ctypes.c_void_p)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python block_quantized_weight_nq_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        L.nq_format_count.restype = c.c_int
        L.nq_format_by_id.argtypes = [c.c_int32, c.POINTER(FormatInfo)]
        L.nq_format_query.argtypes = [c.c_char_p, c.POINTER(FormatInfo)]
        L.nq_validate.argtypes = [c.c_int32, c.c_uint64, c.POINTER(c.c_int64), c.c_int32, c.c_int32,
                                  c.POINTER(c.c_uint64), c.POINTER(c.c_uint64)]
        L.nq_dequantize_packed.argtypes = [c.c_int32, c.c_void_p, c.c_uint64, c.POINTER(c.c_int64),
                                           c.c_int32, c.c_int32, c.c_void_p, c.c_void_p]
        L.nq_dequantize_packed_many.argtypes = [c.POINTER(TensorDesc), c.c_int32, c.c_int32, c.POINTER(c.c_int32),
                                                c.c_void_p]
        L.nq_measure_stream.argtypes = [c.c_void_p, c.c_uint64, c.c_void_p, c.c_uint64, c.c_int32, c.c_int32,
                                        c.c_void_p]
        L.nq_validate_nvfp4_stacked.argtypes = [c.c_uint64, c.POINTER(c.c_int64), c.c_int32, c.c_int64,
                                                c.c_int32, c.POINTER(c.c_uint64), c.POINTER(c.c_uint64)]
        L.nq_dequantize_nvfp4_stacked.argtypes = [c.c_void_p, c.c_uint64, c.POINTER(c.c_int64), c.c_int32,
                                                  c.c_int64, c.c_int32, c.c_void_p, c.c_void_p]
        L.nq_validate_fp8_row.argtypes = [c.c_int32, c.c_uint64, c.POINTER(c.c_int64), c.c_int32, c.c_int32,
                                          c.POINTER(c.c_uint64), c.POINTER(c.c_uint64)]
        L.nq_dequantize_fp8_row.argtypes = [c.c_int32, c.c_void_p, c.c_uint64, c.POINTER(c.c_int64), c.c_int32,
                                            c.c_int32, c.c_void_p, c.c_void_p]
        L.nq_validate_grouped_absmax.argtypes = [c.c_int32, c.POINTER(c.c_int64), c.c_int32, c.c_int32,
                                                 c.POINTER(c.c_uint64), c.POINTER(c.c_uint64)]
        L.nq_quantize_grouped_absmax.argtypes = [c.c_int32, c.c_void_p, c.POINTER(c.c_int64), c.c_int32, c.c_int32,
                                                 c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p]
        L.nq_validate_quantize_q8_1.argtypes = [c.POINTER(c.c_int64), c.c_int32, c.c_int32, c.POINTER(c.c_uint64)]
        L.nq_quantize_q8_1.argtypes = [c.c_void_p, c.POINTER(c.c_int64), c.c_int32, c.c_int32, c.c_void_p,
                                       c.c_void_p, c.c_void_p]
        L.nq_validate_gemv_q8_1.argtypes = [c.c_int32, c.c_uint64, c.c_int64, c.c_int64, c.c_int64]
        L.nq_gemv_q8_1.argtypes = [c.c_int32, c.c_void_p, c.c_uint64, c.c_int64, c.c_int64, c.c_void_p,
                                   c.c_int64, c.c_void_p, c.c_void_p]
        L.nq_validate_gemm_q8_1.argtypes = [c.c_int32, c.c_uint64, c.c_int64, c.c_int64, c.c_int64]
        L.nq_gemm_q8_1_workspace.argtypes = [c.c_int32, c.c_int64, c.c_int64, c.c_int64, c.POINTER(c.c_uint64)]
        L.nq_gemm_q8_1.argtypes = [c.c_int32, c.c_void_p, c.c_uint64, c.c_int64, c.c_int64, c.c_void_p,
                                   c.c_int64, c.c_void_p, c.c_void_p, c.c_uint64, c.c_void_p]
        L.nq_gemm_q8_1_noalloc.argtypes = [c.c_int32, c.c_void_p, c.c_uint64, c.c_int64, c.c_int64, c.c_void_p,
                                            c.c_int64, c.c_void_p, c.c_void_p]
        L.nq_status_string.argtypes = [c.c_int]
        L.nq_status_string.restype = c.c_char_p
        _LIB = L
    return _LIB


def library():
    """The loaded ctypes library (raises if not built)."""
    return _lib()


def format_count():
    return _lib().nq_format_count()


def format_by_id(i):
    info = FormatInfo()
    st = _lib().nq_format_by_id(i, ctypes.byref(info))
    if st != NQ_OK:
        raise NqError(st, f"id {i}")
    return info


def format_query(name):
    info = FormatInfo()
    st = _lib().nq_format_query(name.encode(), ctypes.byref(info))
    if st != NQ_OK:
        raise NqError(st, repr(name))
    return info


def format_names():
    return [format_by_id(i).name.decode() for i in range(format_count())]


def _shape(shape):
    shape = [int(d) for d in shape]
    return (ctypes.c_int64 * max(1, len(shape)))(*shape), len(shape)


def _dtype_code(dtype):
    if isinstance(dtype, str):
        return DTYPE_CODES[dtype]
    import torch
    return {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3}[dtype]


def validate_status(fmt, nbytes, shape, out_dtype="f32"):
    """Raw status of nq_validate plus (elems, out_bytes)."""
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    arr, rank = _shape(shape)
    ne, nb = ctypes.c_uint64(), ctypes.c_uint64()
    code = out_dtype if isinstance(out_dtype, int) else _dtype_code(out_dtype)
    st = _lib().nq_validate(fid, nbytes, arr, rank, code, ctypes.byref(ne), ctypes.byref(nb))
    return st, ne.value, nb.value


def validate(fmt, nbytes, shape, out_dtype="f32"):
    st, ne, nb = validate_status(fmt, nbytes, shape, out_dtype)
    if st != NQ_OK:
        raise NqError(st)
    return ne, nb


def dequantize_packed_raw(fmt_id, payload_ptr, nbytes, shape, out_dtype_code, out_ptr, stream_handle):
    """Direct call of the C entry point with integer addresses; returns the status."""
    arr, rank = _shape(shape)
    return _lib().nq_dequantize_packed(fmt_id, ctypes.c_void_p(payload_ptr), nbytes, arr, rank,
                                       out_dtype_code, ctypes.c_void_p(out_ptr),
                                       ctypes.c_void_p(stream_handle))


class ManyCall:
    """A prepared nq_dequantize_packed_many call: the tensor array is built
    once and reused by every run(stream_handle) (argument marshalling only).
    descs: (format id, payload address, nbytes, shape, out address) per tensor."""

    def __init__(self, descs, out_dtype_code):
        self.n = len(descs)
        self.code = int(out_dtype_code)
        self.arr = (TensorDesc * max(1, self.n))()
        self._shapes = []
        for i, (fid, p, nbytes, shape, o) in enumerate(descs):
            sh, rank = _shape(shape)
            self._shapes.append(sh)
            self.arr[i] = TensorDesc(int(fid), rank, ctypes.cast(sh, ctypes.POINTER(ctypes.c_int64)),
                                     ctypes.c_void_p(p), int(nbytes), ctypes.c_void_p(o))
        self.failed = ctypes.c_int32(-1)

    def run_status(self, stream_handle):
        st = _lib().nq_dequantize_packed_many(self.arr if self.n else None, self.n, self.code,
                                              ctypes.byref(self.failed), ctypes.c_void_p(stream_handle))
        return st, self.failed.value

    def run(self, stream_handle):
        st, failed = self.run_status(stream_handle)
        if st != NQ_OK:
            raise NqError(st, f"tensor {failed}")


def dequantize_packed_many_raw(descs, out_dtype_code, stream_handle):
    """Direct call of nq_dequantize_packed_many.  descs: (format id, payload
    address, nbytes, shape, out address) per tensor.  Returns (status, index
    of the failing tensor or -1)."""
    return ManyCall(descs, out_dtype_code).run_status(stream_handle)


def dequantize_packed_many(items, out_dtype=None, stream=None):
    """Decode several tensors in as few launches as their formats allow.

    items: (fmt, payload, shape) or (fmt, payload, shape, out) per tensor, with
    payload a rank-1 uint8 CUDA tensor.  Returns the output tensors (new ones
    where out is not given), decoded on `stream` (default: the current stream).
    """
    import torch
    descs, outs = [], []
    for it in items:
        fmt, payload, shape = it[0], it[1], it[2]
        out = it[3] if len(it) > 3 else None
        fid = fmt if isinstance(fmt, int) else format_query(fmt).id
        code, out, stream = _prepare(payload, shape, out_dtype if out_dtype is not None else
                                     (out.dtype if out is not None else torch.float32), out, stream)
        descs.append((fid, payload.data_ptr(), payload.numel(), shape, out.data_ptr()))
        outs.append(out)
    if stream is None:
        stream = torch.cuda.current_stream()
    if out_dtype is None:
        out_dtype = outs[0].dtype if outs else torch.float32
    st, failed = dequantize_packed_many_raw(descs, _dtype_code(out_dtype), stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"tensor {failed}")
    return outs


STREAM_NT_LOAD, STREAM_NT_STORE = 1, 2


def measure_stream_raw(src_ptr, src_bytes, dst_ptr, dst_bytes, chunks_per_thread, flags, stream_handle):
    """nq_measure_stream (measurement aid): read src_bytes, write dst_bytes; returns the status."""
    return _lib().nq_measure_stream(ctypes.c_void_p(src_ptr), int(src_bytes), ctypes.c_void_p(dst_ptr),
                                    int(dst_bytes), int(chunks_per_thread), int(flags),
                                    ctypes.c_void_p(stream_handle))


def validate_nvfp4_stacked_status(nbytes, shape, divisors, out_dtype="f32"):
    """Raw status of nq_validate_nvfp4_stacked plus (elems, out_bytes)."""
    arr, rank = _shape(shape)
    ne, nb = ctypes.c_uint64(), ctypes.c_uint64()
    code = out_dtype if isinstance(out_dtype, int) else _dtype_code(out_dtype)
    st = _lib().nq_validate_nvfp4_stacked(nbytes, arr, rank, int(divisors), code, ctypes.byref(ne),
                                          ctypes.byref(nb))
    return st, ne.value, nb.value


def dequantize_nvfp4_stacked_raw(payload_ptr, nbytes, shape, divisors, out_dtype_code, out_ptr, stream_handle):
    """Direct call of nq_dequantize_nvfp4_stacked with integer addresses; returns the status."""
    arr, rank = _shape(shape)
    return _lib().nq_dequantize_nvfp4_stacked(ctypes.c_void_p(payload_ptr), nbytes, arr, rank, int(divisors),
                                              out_dtype_code, ctypes.c_void_p(out_ptr),
                                              ctypes.c_void_p(stream_handle))


def _prepare(payload, shape, out_dtype, out, stream):
    import torch
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    code = _dtype_code(out_dtype)
    if payload.dtype != torch.uint8 or payload.dim() != 1 or not payload.is_cuda:
        raise ValueError("payload must be a rank-1 torch.uint8 CUDA tensor")
    if not payload.is_contiguous():
        raise ValueError("payload must be contiguous")
    n = 1
    for d in shape:
        n *= int(d)
    if out is None:
        out = torch.empty([int(d) for d in shape], dtype=out_dtype, device=payload.device)
    elif (out.dtype != out_dtype or not out.is_contiguous() or out.numel() != n or
          (n and out.device != payload.device)):
        raise ValueError("out must be a contiguous tensor of the requested dtype, size and device")
    if stream is None:
        stream = torch.cuda.current_stream(payload.device)
    return code, out, stream


def dequantize_nvfp4_stacked(payload, shape, divisors, out_dtype=None, out=None, stream=None):
    """Decode an "nvfp4" plane stacked from `divisors` sources (one binary32
    divisor per source after the blocks) into a new (or the given) tensor."""
    code, out, stream = _prepare(payload, shape, out_dtype, out, stream)
    st = dequantize_nvfp4_stacked_raw(payload.data_ptr(), payload.numel(), shape, divisors, code,
                                      out.data_ptr(), stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"nvfp4 {list(shape)} divisors={divisors}")
    return out


def validate_fp8_row_status(fmt, nbytes, shape, out_dtype="f32"):
    """Raw status of nq_validate_fp8_row plus (elems, out_bytes); fmt is the
    format name or the scale kind (0 bf16 scales, 1 fp16 scales)."""
    kind = FP8_ROW_KINDS[fmt] if isinstance(fmt, str) else int(fmt)
    arr, rank = _shape(shape)
    ne, nb = ctypes.c_uint64(), ctypes.c_uint64()
    code = out_dtype if isinstance(out_dtype, int) else _dtype_code(out_dtype)
    st = _lib().nq_validate_fp8_row(kind, nbytes, arr, rank, code, ctypes.byref(ne), ctypes.byref(nb))
    return st, ne.value, nb.value


def dequantize_fp8_row_raw(kind, payload_ptr, nbytes, shape, out_dtype_code, out_ptr, stream_handle):
    """Direct call of nq_dequantize_fp8_row with integer addresses; returns the status."""
    arr, rank = _shape(shape)
    return _lib().nq_dequantize_fp8_row(int(kind), ctypes.c_void_p(payload_ptr), nbytes, arr, rank, out_dtype_code,
                                        ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream_handle))


def dequantize_fp8_row(fmt, payload, shape, out_dtype=None, out=None, stream=None):
    """Decode a row-scaled FP8 matrix ("fp8_e4m3fn_row_bf16" or "_fp16":
    N*K codes, then N scale words) into a new (or the given) [N, K] tensor."""
    code, out, stream = _prepare(payload, shape, out_dtype, out, stream)
    st = dequantize_fp8_row_raw(FP8_ROW_KINDS[fmt], payload.data_ptr(), payload.numel(), shape, code,
                                out.data_ptr(), stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"{fmt} {list(shape)}")
    return out


def validate_grouped_absmax_status(scheme, shape, in_dtype="f32"):
    """Raw status of nq_validate_grouped_absmax plus (codes bytes, scales bytes)."""
    sid = GQ_SCHEMES[scheme][0] if isinstance(scheme, str) else int(scheme)
    arr, rank = _shape(shape)
    cb, sb = ctypes.c_uint64(), ctypes.c_uint64()
    code = in_dtype if isinstance(in_dtype, int) else _dtype_code(in_dtype)
    st = _lib().nq_validate_grouped_absmax(sid, arr, rank, code, ctypes.byref(cb), ctypes.byref(sb))
    return st, cb.value, sb.value


def quantize_grouped_absmax_raw(scheme_id, x_ptr, shape, in_dtype_code, codes_ptr, scales_ptr, status_ptr,
                                stream_handle):
    """Direct call of nq_quantize_grouped_absmax with integer addresses; returns the status."""
    arr, rank = _shape(shape)
    return _lib().nq_quantize_grouped_absmax(int(scheme_id), ctypes.c_void_p(x_ptr), arr, rank, in_dtype_code,
                                             ctypes.c_void_p(codes_ptr), ctypes.c_void_p(scales_ptr),
                                             ctypes.c_void_p(status_ptr), ctypes.c_void_p(stream_handle))


def quantize_grouped_absmax(scheme, x, stream=None, check=True):
    """Encode a contiguous [N, K] CUDA tensor (float32/float16/bfloat16/float64)
    with grouped_absmax.  Returns (codes int8 [N, K], scales as int16 words
    [N, ceil(K/G)], status int32 [1]).  With check=True the call waits for
    the stream and raises NqError-like ValueError on an encoder failure."""
    import torch
    sid, G = GQ_SCHEMES[scheme]
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous rank-2 CUDA tensor")
    N, K = x.shape
    codes = torch.empty((N, K), dtype=torch.int8, device=x.device)
    scales = torch.empty((N, (K + G - 1) // G), dtype=torch.int16, device=x.device)
    status = torch.empty(1, dtype=torch.int32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = quantize_grouped_absmax_raw(sid, x.data_ptr(), [N, K], _dtype_code(x.dtype), codes.data_ptr(),
                                     scales.data_ptr(), status.data_ptr(), stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"{scheme} {[N, K]}")
    if check:
        stream.synchronize()
        bits = int(status.item())
        if bits:
            raise ValueError(f"grouped_absmax failed: status bits {bits:#x} "
                             "(1: a source value is not finite, 2: a scale rounds past binary16)")
    return codes, scales, status


def validate_quantize_q8_1_status(shape, in_dtype="f32"):
    """Raw status of nq_validate_quantize_q8_1 plus the blocks' byte size."""
    arr, rank = _shape(shape)
    nb = ctypes.c_uint64()
    code = in_dtype if isinstance(in_dtype, int) else _dtype_code(in_dtype)
    st = _lib().nq_validate_quantize_q8_1(arr, rank, code, ctypes.byref(nb))
    return st, nb.value


def quantize_q8_1_raw(x_ptr, shape, in_dtype_code, blocks_ptr, status_ptr, stream_handle):
    """Direct call of nq_quantize_q8_1 with integer addresses; returns the status."""
    arr, rank = _shape(shape)
    return _lib().nq_quantize_q8_1(ctypes.c_void_p(x_ptr), arr, rank, in_dtype_code, ctypes.c_void_p(blocks_ptr),
                                   ctypes.c_void_p(status_ptr), ctypes.c_void_p(stream_handle))


def quantize_q8_1(x, stream=None, check=True):
    """q8_1 activation blocks of a contiguous [M, K] CUDA tensor (float32 /
    float16 / bfloat16 / float64, K % 32 == 0).  Returns (blocks uint8
    [M, K/32, 36], status int32 [1]).  With check=True the call waits for the
    stream and raises ValueError on a non-finite source or a scale past
    binary16."""
    import torch
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous rank-2 CUDA tensor")
    M, K = x.shape
    blocks = torch.empty((M, K // 32, 36), dtype=torch.uint8, device=x.device)
    status = torch.empty(1, dtype=torch.int32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = quantize_q8_1_raw(x.data_ptr(), [M, K], _dtype_code(x.dtype), blocks.data_ptr(), status.data_ptr(),
                           stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"q8_1 {[M, K]}")
    if check:
        stream.synchronize()
        bits = int(status.item())
        if bits & 3:
            raise ValueError(f"q8_1 quantization failed: status bits {bits:#x} "
                             "(1: a source value is not finite, 2: a scale rounds past binary16)")
    return blocks, status


def validate_gemv_q8_1_status(fmt, nbytes, N, K, M):
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    return _lib().nq_validate_gemv_q8_1(fid, nbytes, N, K, M)


def gemv_q8_1_raw(fmt_id, w_ptr, nbytes, N, K, xq_ptr, M, y_ptr, stream_handle):
    """Direct call of nq_gemv_q8_1 with integer addresses; returns the status."""
    return _lib().nq_gemv_q8_1(int(fmt_id), ctypes.c_void_p(w_ptr), nbytes, N, K, ctypes.c_void_p(xq_ptr), M,
                               ctypes.c_void_p(y_ptr), ctypes.c_void_p(stream_handle))


def validate_gemm_q8_1_status(fmt, nbytes, N, K, M):
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    return _lib().nq_validate_gemm_q8_1(fid, nbytes, N, K, M)


def gemm_q8_1_workspace(fmt, N, K, M):
    """(status, workspace bytes) of the batched product for this shape on the current device."""
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    b = ctypes.c_uint64(0)
    st = _lib().nq_gemm_q8_1_workspace(fid, N, K, M, ctypes.byref(b))
    return st, b.value


def gemm_q8_1_raw(fmt_id, w_ptr, nbytes, N, K, xq_ptr, M, y_ptr, ws_ptr, ws_bytes, stream_handle):
    """Direct call of nq_gemm_q8_1 with integer addresses; returns the status."""
    return _lib().nq_gemm_q8_1(int(fmt_id), ctypes.c_void_p(w_ptr), nbytes, N, K, ctypes.c_void_p(xq_ptr), M,
                               ctypes.c_void_p(y_ptr), ctypes.c_void_p(ws_ptr), ws_bytes,
                               ctypes.c_void_p(stream_handle))


GEMM_SCRATCH_BYTES = 32 << 20


def gemm_q8_1_noalloc_raw(fmt_id, w_ptr, nbytes, N, K, xq_ptr, M, y_ptr, stream_handle):
    """nq_gemm_q8_1_noalloc (the library's static scratch as the workspace); returns the status."""
    return _lib().nq_gemm_q8_1_noalloc(fmt_id, ctypes.c_void_p(w_ptr), nbytes, N, K, ctypes.c_void_p(xq_ptr), M,
                                       ctypes.c_void_p(y_ptr), ctypes.c_void_p(stream_handle))


def _product(raw, fmt, weight, N, K, xq, out, stream):
    import torch
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    if not weight.is_cuda or not xq.is_cuda or xq.dtype != torch.uint8 or not xq.is_contiguous():
        raise ValueError("weight and xq must be CUDA uint8 tensors, xq contiguous")
    M = xq.numel() // (K // 32 * 36) if K % 32 == 0 and K > 0 else 0
    if xq.numel() != M * (K // 32) * 36:
        raise ValueError("xq holds a whole number of activation rows of K / 32 blocks")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=weight.device)
    elif out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != M * N:
        raise ValueError("out must be a contiguous float32 tensor of M * N elements")
    if stream is None:
        stream = torch.cuda.current_stream(weight.device)
    st = raw(fid, weight.data_ptr(), weight.numel(), N, K, xq.data_ptr(), M, out.data_ptr(), stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"{fmt} [{N}, {K}] x {M}")
    return out


def gemv_q8_1(fmt, weight, N, K, xq, out=None, stream=None):
    """y[M, N] (float32) = x[M, K] @ w[N, K]^T for a rank-1 uint8 CUDA weight
    payload of `fmt` (a "gguf:" format) and q8_1 activation blocks `xq`
    ([M, K/32, 36] uint8, as quantize_q8_1 returns), M <= 8."""
    return _product(gemv_q8_1_raw, fmt, weight, N, K, xq, out, stream)


def gemm_q8_1(fmt, weight, N, K, xq, out=None, stream=None, split=True):
    """As gemv_q8_1 for any number of activation rows M >= 1 (5 or more on
    the matrix cores).  With split=True the workspace the product may use is
    allocated from torch on `stream` (K then splits, and the weight is
    rewritten once, where the shape asks for it); split=False runs without a
    workspace."""
    import torch
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    M = xq.numel() // (K // 32 * 36) if K % 32 == 0 and K > 0 else 0
    ws, ws_bytes = None, 0
    if split and M > 0:
        st, ws_bytes = gemm_q8_1_workspace(fid, N, K, M)
        if st != NQ_OK:
            raise NqError(st, f"{fmt} [{N}, {K}] x {M}")
        if ws_bytes:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=weight.device)
            if stream is not None:
                ws.record_stream(stream)

    def raw(fid_, w_ptr, nbytes, N_, K_, xq_ptr, M_, y_ptr, h):
        return gemm_q8_1_raw(fid_, w_ptr, nbytes, N_, K_, xq_ptr, M_, y_ptr, ws.data_ptr() if ws is not None else 0,
                             ws_bytes, h)

    return _product(raw, fmt, weight, N, K, xq, out, stream)


def dequantize_packed(fmt, payload, shape, out_dtype=None, out=None, stream=None):
    """Decode a rank-1 uint8 CUDA tensor into a new (or the given) tensor of `shape`.

    out_dtype: torch.float32 (default), torch.float16, torch.bfloat16 or torch.float64.
    The decode is enqueued on `stream` (default: the current stream).
    """
    fid = fmt if isinstance(fmt, int) else format_query(fmt).id
    code, out, stream = _prepare(payload, shape, out_dtype, out, stream)
    st = dequantize_packed_raw(fid, payload.data_ptr(), payload.numel(), shape, code,
                               out.data_ptr(), stream.cuda_stream)
    if st != NQ_OK:
        raise NqError(st, f"{fmt} {list(shape)}")
    return out
