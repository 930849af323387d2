"""Build and call the host emulator of the decode kernels (tests/emu/nq_emu.hip)."""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "emu", "nq_emu.hip")
LIB = os.path.join(HERE, "emu", "libnq_emu.so")
CSRC = os.path.join(os.path.dirname(HERE), "block_quantized_weight_nq_amd", "csrc")
OSIZE = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8}
NPT = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}
_lib = None


PARTS = 6


# NQ_EMU_DEFINES="NAME=VALUE ..." builds and loads an emulator with the
# kernels' tuning knobs set (a separate library file), to check the code
# paths a tuning choice selects.
DEFINES = os.environ.get("NQ_EMU_DEFINES", "").split()
if DEFINES:
    LIB = os.path.join(HERE, "emu", "libnq_emu_" + "_".join(d.replace("=", "") for d in DEFINES) + ".so")
# NQ_SANITIZE=1: host code under AddressSanitizer and UndefinedBehaviorSanitizer
# (tests/run_sanitized.py preloads the runtime)
SANITIZE = os.environ.get("NQ_SANITIZE") == "1"
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
if SANITIZE:
    LIB = LIB[:-3] + "_san.so"


def build():
    """Compile the emulator: PARTS instantiation parts and the dispatch part in parallel, then link."""
    import concurrent.futures
    import tempfile
    flags = ["hipcc", "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-fvisibility=hidden"] + [f"-D{d}" for d in DEFINES] + (SAN_FLAGS if SANITIZE else [])
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [[f"-DNQ_EMU_PART={p}", f"-DNQ_EMU_PARTS={PARTS}"] for p in range(PARTS)] + [[]]
        objs = [os.path.join(tmp, f"part{i}.o") for i in range(len(jobs))]

        def compile_one(i):
            return subprocess.run(flags + jobs[i] + ["-c", SRC, "-o", objs[i]], capture_output=True, text=True)

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
            results = list(ex.map(compile_one, range(len(jobs))))
        for r in results:
            if r.returncode != 0:
                raise RuntimeError(f"emulator build failed:\n{r.stderr[-4000:]}")
        part = LIB + f".{os.getpid()}.tmp"  # linked next to LIB, then renamed onto it (atomic)
        subprocess.run(["hipcc", "-shared", "-fPIC"] + objs + ["-o", part], check=True, capture_output=True)
        os.replace(part, LIB)


def _stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [SRC] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    return any(os.path.getmtime(d) > t for d in deps)


def lib():
    global _lib
    if _lib is None:
        if _stale():
            import fcntl
            with open(LIB + ".lock", "w") as lk:  # one builder among parallel test processes
                fcntl.flock(lk, fcntl.LOCK_EX)
                if _stale():
                    build()
        L = ctypes.CDLL(LIB)
        L.nq_emu_decode.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                                    ctypes.c_int, ctypes.c_uint32, ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_decode.restype = ctypes.c_long
        L.nq_emu_decode_many.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                                         ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                         ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_decode_many.restype = ctypes.c_long
        L.nq_emu_nvfp4_tables.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p]
        L.nq_emu_nvfp4_tables.restype = None
        L.nq_emu_tile_blocks.argtypes = [ctypes.c_int, ctypes.c_int]
        L.nq_emu_fp8_row.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_void_p, ctypes.c_uint64, ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_fp8_row.restype = ctypes.c_long
        L.nq_emu_f8_div.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.nq_emu_grouped_absmax.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64,
                                            ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_grouped_absmax.restype = ctypes.c_long
        L.nq_emu_f8_div.restype = ctypes.c_uint32
        L.nq_emu_kq_scale_min_pair.argtypes = [ctypes.c_uint32] * 4
        L.nq_emu_kq_scale_min_pair.restype = ctypes.c_uint32
        L.nq_emu_choose_upt.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32]
        L.nq_emu_choose_upt.restype = ctypes.c_int
        L.nq_emu_tile_blocks.restype = ctypes.c_long
        L.nq_emu_gemv_q8_1.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32,
                                       ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                       ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_gemv_q8_1.restype = ctypes.c_long
        L.nq_emu_gemv1_plan.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        L.nq_emu_gemv1_plan.restype = ctypes.c_int
        L.nq_emu_gemm_q8_1.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32),
                                       ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_gemm_q8_1.restype = ctypes.c_long
        L.nq_emu_gemm_plan.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_uint32, ctypes.c_void_p]
        L.nq_emu_gemm_plan.restype = None
        L.nq_emu_quantize_q8_1.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_uint64, ctypes.c_char_p, ctypes.c_int]
        L.nq_emu_quantize_q8_1.restype = ctypes.c_long
        _lib = L
    return _lib


def _placed(nbytes, align, mis, slack=64):
    """A uint8 buffer and an offset whose address is `mis` mod `align`."""
    buf = np.zeros(nbytes + 2 * slack + align, dtype=np.uint8)
    base = buf.ctypes.data
    off = slack + ((mis - (base + slack)) % align)
    return buf, off


def decode(fmt_id, payload, nblocks, B, dtype, mis=0, out_mis=0, max_wgs=2048, chunk=0, upt=0, ndiv=1):
    """Run the emulator; returns (values, out-of-payload reads, message, guards_ok)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    pbuf, poff = _placed(payload.size, 4, mis)
    pbuf[:] = 0xEE
    pbuf[poff:poff + payload.size] = payload
    n = nblocks * B
    osz = OSIZE[dtype]
    obuf, ooff = _placed(n * osz, 16, out_mis)
    obuf[:] = 0xA5
    err = ctypes.create_string_buffer(256)
    rc = lib().nq_emu_decode(fmt_id, {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}[dtype],
                             pbuf.ctypes.data + poff, payload.size, nblocks,
                             obuf.ctypes.data + ooff, max_wgs, chunk, upt, ndiv, err, 256)
    guards = bool(np.all(obuf[:ooff] == 0xA5) and np.all(obuf[ooff + n * osz:] == 0xA5))
    vals = obuf[ooff:ooff + n * osz].copy().view(NPT[dtype])
    return vals, rc, err.value.decode(), guards


def decode_many(fmt_id, payloads, B, dtype, vec=True, resident=2048, chunk=0, mis=0):
    """Many-tensor decode of payloads (one format; each payload whole blocks plus
    its trailer) through the emulator.  Outputs are 16-byte aligned (vec) or
    shifted by one element.  Returns (values per tensor, errors, message,
    guards_ok, launches, set of units-per-thread taken)."""
    osz = OSIZE[dtype]
    bufs, outs, pptr, nbytes, nblocks, optr = [], [], [], [], [], []
    info = _format(fmt_id)
    T = info.trailer_bytes
    for k, p in enumerate(payloads):
        p = np.ascontiguousarray(p, dtype=np.uint8)
        pb, po = _placed(p.size, 4, (mis + k) % 4)
        pb[:] = 0xEE
        pb[po:po + p.size] = p
        nb = (p.size - T) // info.block_bytes
        n = nb * B
        ob, oo = _placed(n * osz, 16, 0 if vec else osz)
        ob[:] = 0xA5
        bufs.append((pb, po))
        outs.append((ob, oo, n))
        pptr.append(pb.ctypes.data + po)
        nbytes.append(p.size)
        nblocks.append(nb)
        optr.append(ob.ctypes.data + oo)
    cnt = len(payloads)
    arr_p = (ctypes.c_void_p * max(1, cnt))(*pptr)
    arr_nb = (ctypes.c_uint64 * max(1, cnt))(*nbytes)
    arr_bl = (ctypes.c_uint64 * max(1, cnt))(*nblocks)
    arr_o = (ctypes.c_void_p * max(1, cnt))(*optr)
    err = ctypes.create_string_buffer(256)
    launches, mask = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib().nq_emu_decode_many(fmt_id, {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}[dtype], cnt, arr_p, arr_nb,
                                  arr_bl, arr_o, resident, chunk, ctypes.byref(launches), ctypes.byref(mask), err, 256)
    vals, guards = [], True
    for ob, oo, n in outs:
        guards &= bool(np.all(ob[:oo] == 0xA5) and np.all(ob[oo + n * osz:] == 0xA5))
        vals.append(ob[oo:oo + n * osz].copy().view(NPT[dtype]))
    upts = {u for u in (1, 2, 4, 8, 16) if mask.value >> u & 1}
    return vals, rc, err.value.decode(), guards, launches.value, upts


def _format(fmt_id):
    import block_quantized_weight_nq_amd as nq
    return nq.format_by_id(fmt_id)


def nvfp4_tables(dw_bits):
    """(quad-built, entry-built) nvfp4 quotient tables, [n, 1024] uint32 each."""
    dw_bits = np.ascontiguousarray(dw_bits, dtype=np.uint32)
    n = dw_bits.size
    quad = np.zeros((n, 1024), dtype=np.uint32)
    direct = np.zeros((n, 1024), dtype=np.uint32)
    lib().nq_emu_nvfp4_tables(dw_bits.ctypes.data, n, quad.ctypes.data, direct.ctypes.data)
    return quad, direct


def tile_blocks(fmt_id, upt):
    """Whole blocks per staged tile of the format's kernel at `upt` units per thread."""
    return lib().nq_emu_tile_blocks(fmt_id, upt)


def choose_upt(fmt_id, nunits, resident):
    """The launcher's units per thread for a launch of `nunits` units of a format."""
    return lib().nq_emu_choose_upt(fmt_id, nunits, resident)


def decode_fp8_row(kind, payload, N, K, dtype, mis=0, out_mis=0, chunk=0):
    """Row-scaled FP8 through the emulator; returns (values, out-of-bounds reads, message, guards_ok)."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8)
    pbuf, poff = _placed(payload.size, 4, mis)
    pbuf[:] = 0xEE
    pbuf[poff:poff + payload.size] = payload
    n = N * K
    osz = OSIZE[dtype]
    obuf, ooff = _placed(n * osz, 16, out_mis)
    obuf[:] = 0xA5
    err = ctypes.create_string_buffer(256)
    rc = lib().nq_emu_fp8_row(kind, {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}[dtype], pbuf.ctypes.data + poff, N, K,
                              obuf.ctypes.data + ooff, chunk, err, 256)
    guards = bool(np.all(obuf[:ooff] == 0xA5) and np.all(obuf[ooff + n * osz:] == 0xA5))
    vals = obuf[ooff:ooff + n * osz].copy().view(NPT[dtype])
    return vals, rc, err.value.decode(), guards


def f8_div(n, d):
    """The FP8 row kernels' multiply-shift division floor(n / d)."""
    return lib().nq_emu_f8_div(n, d)


def kq_scale_min_pair(scales12, g):
    """The product's sub-scale and min pair of 64-value item g (< 4) of a
    K-quant block from its 12 packed scale bytes: (sc(2g), sc(2g+1), m(2g),
    m(2g+1))."""
    h = np.frombuffer(bytes(scales12), dtype="<u4")
    w = lib().nq_emu_kq_scale_min_pair(int(h[0]), int(h[1]), int(h[2]), g)
    return tuple((w >> (8 * k)) & 0xFF for k in range(4))


def grouped_absmax(scheme_id, G, x, in_code, x_mis=0, codes_mis=0):
    """The encoder through the emulator.  x: [N, K] array (raw words for
    f16/bf16).  Returns (status, codes, scales, bad reads, message, guards_ok)."""
    x = np.ascontiguousarray(x)
    N, K = x.shape
    xbuf, xoff = _placed(x.nbytes, 16, x_mis)
    xbuf[xoff:xoff + x.nbytes] = x.view(np.uint8).ravel()
    cbuf, coff = _placed(N * K, 16, codes_mis)
    cbuf[:] = 0xA5
    ng = (K + G - 1) // G
    sbuf = np.full(N * ng + 16, 0xA5A5, dtype=np.uint16)
    status = np.zeros(1, dtype=np.uint32)
    err = ctypes.create_string_buffer(256)
    rc = lib().nq_emu_grouped_absmax(scheme_id, in_code, xbuf.ctypes.data + xoff, N, K, cbuf.ctypes.data + coff,
                                     sbuf.ctypes.data + 16, status.ctypes.data, err, 256)
    guards = bool(np.all(cbuf[:coff] == 0xA5) and np.all(cbuf[coff + N * K:] == 0xA5) and
                  np.all(sbuf[:8] == 0xA5A5) and np.all(sbuf[8 + N * ng:] == 0xA5A5))
    codes = cbuf[coff:coff + N * K].view(np.int8).reshape(N, K).copy()
    scales = sbuf[8:8 + N * ng].reshape(N, ng).copy()
    return int(status[0]), codes, scales, rc, err.value.decode(), guards


def gemv_q8_1(fmt_id, w, N, K, xq, M, w_mis=0, resident=2048, max_rows=0, gv1_cus=0, gv1_per_cu=8,
              with_rw=False, with_parts=False):
    """The product through the emulator.  w: payload bytes, xq: q8_1 blocks.
    gv1_cus > 0: the launcher's single-round plan on a device of that many
    compute units holding at most gv1_per_cu workgroups each (else, or when
    the plan makes none, the chunk-loop kernel with `resident` workgroups).
    Returns (y float32 [M, N], bad reads, message, guards_ok[, rows per
    single-round chunk or 0][, parts per row of a single-round launch])."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    wbuf, woff = _placed(w.size, 16, w_mis)
    wbuf[woff:woff + w.size] = w
    xq = np.ascontiguousarray(xq, dtype=np.uint8).reshape(-1)
    xbuf, xoff = _placed(xq.size, 16, 0)
    xbuf[xoff:xoff + xq.size] = xq
    ybuf = np.full(M * N + 32, np.float32(np.nan), dtype=np.float32)
    err = ctypes.create_string_buffer(256)
    rw = ctypes.c_uint32(0)
    rc = lib().nq_emu_gemv_q8_1(fmt_id, wbuf.ctypes.data + woff, N, K, xbuf.ctypes.data + xoff, M,
                                ybuf.ctypes.data + 64, resident, max_rows, gv1_cus, gv1_per_cu, ctypes.byref(rw),
                                err, 256)
    y = ybuf[16:16 + M * N].reshape(M, N).copy()
    guards = bool(np.all(np.isnan(ybuf[:16])) and np.all(np.isnan(ybuf[16 + M * N:])))
    out = (y, rc, err.value.decode(), guards)
    if with_rw:
        out += (rw.value & 0xFF,)
    if with_parts:
        out += (rw.value >> 8,)
    return out


def gemv1_plan(fmt_id, N, K, M, w_mis=0, cus=256, per_cu=8):
    """The launcher's single-round product plan on the emulator's device
    model (at most per_cu workgroups, 160 KiB of LDS and 32 waves per compute
    unit): (rows per chunk or 0, region dwords, LDS bytes, workgroups, parts
    per row, blocks per chunk row, waves per workgroup, activation dwords)."""
    out = (ctypes.c_uint64 * 8)()
    rc = lib().nq_emu_gemv1_plan(fmt_id, N, K, M, w_mis, cus, per_cu, out)
    assert rc == 0
    return tuple(int(v) for v in out)


def gemm_q8_1(fmt_id, w, N, K, xq, M, w_mis=0, max_rows=0, max_mrows=0, cus=0, with_splits=False):
    """The matrix-core product through the emulator (cus > 0: a device of
    that many compute units with the workspace its plan asks for: K split,
    and the weight rewritten once per call for more than 64 activation rows;
    0: no workspace).  Returns (y float32 [M, N], bad reads, message,
    guards_ok[, (K splits, rewritten once, 4-span K steps)]); bad reads is
    -1 for a format without a span rewrite."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    wbuf, woff = _placed(w.size, 16, w_mis)
    wbuf[woff:woff + w.size] = w
    xq = np.ascontiguousarray(xq, dtype=np.uint8).reshape(-1)
    xbuf, xoff = _placed(xq.size, 16, 0)
    xbuf[xoff:xoff + xq.size] = xq
    ybuf = np.full(M * N + 32, np.float32(np.nan), dtype=np.float32)
    err = ctypes.create_string_buffer(256)
    ns = ctypes.c_uint32(0)
    rc = lib().nq_emu_gemm_q8_1(fmt_id, wbuf.ctypes.data + woff, N, K, xbuf.ctypes.data + xoff, M,
                                ybuf.ctypes.data + 64, max_rows, max_mrows, cus, ctypes.byref(ns), err, 256)
    y = ybuf[16:16 + M * N].reshape(M, N).copy()
    guards = bool(np.all(np.isnan(ybuf[:16])) and np.all(np.isnan(ybuf[16 + M * N:])))
    if with_splits:
        return y, rc, err.value.decode(), guards, (ns.value & 0xFFFF, bool(ns.value >> 16 & 1),
                                                   bool(ns.value >> 17 & 1))
    return y, rc, err.value.decode(), guards


def gemm_plan(fmt_id, N, K, M, cus):
    """The batched product's plan on `cus` compute units: a dict of nsplit,
    sps (steps per split), sp (spans per step), once (weight rewritten once),
    bm (tile height), ws (workspace bytes) and, without a workspace, the
    plain plan's nsplit, sps and sp (plain_*)."""
    out = np.zeros(9, dtype=np.uint64)
    lib().nq_emu_gemm_plan(fmt_id, N, K, M, cus, out.ctypes.data)
    keys = ["nsplit", "sps", "sp", "once", "bm", "ws", "plain_nsplit", "plain_sps", "plain_sp"]
    return {k: int(v) for k, v in zip(keys, out)}


def quantize_q8_1(x, in_code, x_mis=0, chunk=0):
    """The q8_1 quantizer through the emulator.  x: [M, K] array (raw words
    for f16/bf16).  Returns (status, blocks uint8 [M, K/32, 36], bad reads,
    message, guards_ok)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    xbuf, xoff = _placed(x.nbytes, 16, x_mis)
    xbuf[xoff:xoff + x.nbytes] = x.view(np.uint8).ravel()
    nb = M * K // 32
    bbuf = np.full(nb * 9 + 8, 0xA5A5A5A5, dtype=np.uint32)
    status = np.zeros(1, dtype=np.uint32)
    err = ctypes.create_string_buffer(256)
    rc = lib().nq_emu_quantize_q8_1(in_code, xbuf.ctypes.data + xoff, nb, bbuf.ctypes.data + 16,
                                    status.ctypes.data, chunk, err, 256)
    guards = bool(np.all(bbuf[:4] == 0xA5A5A5A5) and np.all(bbuf[4 + nb * 9:] == 0xA5A5A5A5))
    blocks = bbuf[4:4 + nb * 9].view(np.uint8).reshape(M, K // 32, 36).copy()
    return int(status[0]), blocks, rc, err.value.decode(), guards
