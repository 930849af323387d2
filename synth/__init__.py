"""Seeded synthetic payloads for packed block-quantized weights.

A thin ctypes wrapper over ``synth.c``: a counter-based SplitMix64 byte
stream laid out block by block, with each format's scale fields drawn from
the workload recipe (see ``synth.c``).  The module knows where scale fields
sit in a block, never how a block decodes, so it can feed both the HIP path
and the oracle.

Recipes used by the tests and the benchmark (exponent ranges are whole
binades [2**lo, 2**hi)):

* ``raw()``                        every byte uniform;
* ``binade(lo, hi, signed)``       scale fields log-uniform over binades.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SANITIZE = os.environ.get("NQ_SANITIZE") == "1"  # separate sanitized build (tests/run_sanitized.py)
_LIB_PATH = os.path.join(_HERE, "libsynth_san.so" if SANITIZE else "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")
_lib = None


def build():
    """Compile libsynth.so (gcc, OpenMP; NQ_SANITIZE=1: libsynth_san.so, clang with the sanitizers)."""
    if SANITIZE:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
               "-o", _LIB_PATH, _SRC]
    else:
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH, _SRC]
    subprocess.run(cmd, check=True)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.argtypes = [ctypes.c_char_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_block_bytes.argtypes = [ctypes.c_char_p]
        lib.synth_block_bytes.restype = ctypes.c_int
        lib.synth_trailer_bytes.argtypes = [ctypes.c_char_p]
        lib.synth_trailer_bytes.restype = ctypes.c_int
        lib.synth_divisor_bits.argtypes = [ctypes.c_uint64]
        lib.synth_divisor_bits.restype = ctypes.c_uint32
        lib.synth_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint]
        lib.synth_splitmix64.restype = ctypes.c_uint64
        _lib = lib
    return _lib


class Recipe:
    def __init__(self, mode, lo=0, hi=1, signed=False):
        self.mode, self.lo, self.hi, self.signed = mode, lo, hi, signed

    def __repr__(self):
        if self.mode == 0:
            return "raw"
        return f"binade[2^{self.lo},2^{self.hi}){'±' if self.signed else '+'}"


def raw():
    return Recipe(0)


def binade(lo, hi, signed=False):
    return Recipe(1, lo, hi, signed)


def block_bytes(fmt):
    s = _load().synth_block_bytes(fmt.encode())
    if s < 0:
        raise KeyError(fmt)
    return s


def trailer_bytes(fmt):
    return _load().synth_trailer_bytes(fmt.encode())


def divisor_bits(seed):
    return int(_load().synth_divisor_bits(seed))


def splitmix64(seed, block, k):
    return int(_load().synth_splitmix64(seed, block, k))


def fill_into(fmt, nblocks, seed, recipe, buf_ptr):
    """Write nblocks blocks (no trailer) at a host address."""
    rc = _load().synth_fill(fmt.encode(), nblocks, seed, recipe.mode, recipe.lo, recipe.hi,
                            int(recipe.signed), ctypes.c_void_p(buf_ptr))
    if rc != 0:
        raise ValueError(f"synth_fill failed for {fmt}")


def payload(fmt, nblocks, seed, recipe, divisor=None, divisors=1):
    """Return a uint8 array: nblocks blocks, then the trailer if the format has one.

    The trailer of ``nvfp4`` is ``divisors`` little-endian binary32 divisors
    (one per stacked source): ``divisor`` (a float, or a sequence of
    ``divisors`` floats) if given, else bits uniform in [bits(1.0),
    bits(448.0)], the j-th drawn from seed + j.
    """
    S = block_bytes(fmt)
    T = trailer_bytes(fmt)
    nd = divisors if T == 4 else 0
    out = np.empty(nblocks * S + 4 * nd, dtype=np.uint8)
    if nblocks:
        fill_into(fmt, nblocks, seed, recipe, out.ctypes.data)
    if nd:
        if divisor is None:
            bits = [divisor_bits(seed + j) for j in range(nd)]
        else:
            vals = list(divisor) if hasattr(divisor, "__len__") else [divisor] * nd
            assert len(vals) == nd
            bits = [int(v) for v in np.array(vals, dtype=np.float32).view(np.uint32)]
        out[nblocks * S:] = np.array(bits, dtype="<u4").view(np.uint8)
    return out
