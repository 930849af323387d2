"""Bitwise comparison of decoded outputs; NaN compared by class only.

The DequantizePacked page leaves NaN payload bits unspecified, so a NaN
matches any NaN; every other word (signed zeros, subnormals, infinities)
must match bit for bit.
"""
import numpy as np

_MASKS = {"bf16": (0x7F80, 0x007F), "f16": (0x7C00, 0x03FF)}


def nan_mask(x, dtype):
    if dtype in ("f32", "f64"):
        return np.isnan(x)
    e, m = _MASKS[dtype]
    return ((x & e) == e) & ((x & m) != 0)


def mismatches(got, ref, dtype):
    """Indices where got differs from ref under the rule above."""
    gn, rn = nan_mask(got, dtype), nan_mask(ref, dtype)
    if dtype == "f32":
        gw, rw = got.view(np.uint32), ref.view(np.uint32)
    elif dtype == "f64":
        gw, rw = got.view(np.uint64), ref.view(np.uint64)
    else:
        gw, rw = got, ref
    bad = (gn != rn) | (~rn & (gw != rw))
    return np.nonzero(bad)[0]


def same(got, ref, dtype):
    return got.shape == ref.shape and mismatches(got, ref, dtype).size == 0


def describe(got, ref, dtype, limit=5):
    idx = mismatches(got, ref, dtype)
    if idx.size == 0:
        return "ok"
    show = ", ".join(f"[{i}] got {got[i]!r} want {ref[i]!r}" for i in idx[:limit])
    return f"{idx.size} mismatches: {show}"
