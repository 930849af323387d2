"""Pins of the oracle against what the pages and mathematics fix (CPU only).

Each test names the passage it pins.  None of them recomputes the oracle's
own formula: they compare with library routines (numpy, PyTorch), closed
forms, tables printed elsewhere on the pages, hand-derived blocks
(tests/golden/one_block.json), the page's second notation, and a structural
bit-flip map written separately from the layout table (tests/layout_map.py).
"""
import json
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle
import synth
import layout_map
import page_notation

HERE = os.path.dirname(os.path.abspath(__file__))
GGUF = [f for f in oracle.format_names() if f.startswith("gguf:")]
ALL = oracle.format_names()
RECIPE = synth.binade(-12, -6, True)

# --------------------------------------------------------------------------
# Registry: DequantizePacked page, "Quantization formats" (B, S) versus the
# field list of "Packed layouts and decoding" and the NInfer page's GGUF
# bits/weight column.
# --------------------------------------------------------------------------
LAYOUT_FIELDS = {
    "q4_0": "h d; u8 q[16]", "q4_1": "h d,m; u8 q[16]", "q5_0": "h d; u8 high[4],q[16]",
    "q5_1": "h d,m; u8 high[4],q[16]", "q8_0": "h d; i8 q[32]", "q8_1": "h d,s; i8 q[32]",
    "q2_k": "u8 scales[16],q[64]; h d,dmin", "q3_k": "u8 mask[32],q[64],scales[12]; h d",
    "q4_k": "h d,dmin; u8 scales[12],q[128]", "q5_k": "h d,dmin; u8 scales[12],high[32],q[128]",
    "q6_k": "u8 low[128],high[64]; i8 scales[16]; h d", "q8_k": "f d; i8 q[256]; i16 sums[16]",
    "iq2_xxs": "h d; u16 q[32]", "iq2_xs": "h d; u16 q[32]; u8 scales[8]",
    "iq2_s": "h d; u8 q[64],high[8],scales[8]", "iq3_xxs": "h d; u8 q[96]",
    "iq3_s": "h d; u8 q[64],high[8],signs[32],scales[4]", "iq1_s": "h d; u8 q[32]; u16 high[8]",
    "iq1_m": "u8 q[32],high[16],scales[8]", "iq4_nl": "h d; u8 q[16]",
    "iq4_xs": "h d; u16 high; u8 scales[4],q[128]", "tq1_0": "u8 q[48],high[4]; h d",
    "tq2_0": "u8 q[64]; h d", "mxfp4": "u8 exponent,q[16]", "nvfp4": "u8 scales[4],q[32]",
    "q1_0": "h d; u8 q[16]", "q2_0": "h d; u8 q[16]",
}
TYPE_BYTES = {"h": 2, "f": 4, "u8": 1, "i8": 1, "u16": 2, "i16": 2}

# NInfer tensor-formats page, GGUF block format table: name -> (B, S, bits/weight)
NINFER_GGUF = {
    "q8_0": (32, 34, 8.50), "q4_0": (32, 18, 4.50), "q5_0": (32, 22, 5.50), "q2_0": (64, 18, 2.25),
    "q2_k": (256, 84, 2.625), "q3_k": (256, 110, 3.4375), "q4_k": (256, 144, 4.50),
    "q5_k": (256, 176, 5.50), "q6_k": (256, 210, 6.5625), "iq2_xxs": (256, 66, 2.0625),
    "iq2_xs": (256, 74, 2.3125), "iq3_xxs": (256, 98, 3.0625), "iq1_s": (256, 50, 1.5625),
    "iq4_nl": (32, 18, 4.50), "iq3_s": (256, 110, 3.4375), "iq2_s": (256, 82, 2.5625),
    "iq4_xs": (256, 136, 4.25), "iq1_m": (256, 56, 1.75),
}


def _field_bytes(desc):
    total = 0
    for group in desc.split(";"):
        typ, rest = group.strip().split(" ", 1)
        for name in rest.split(","):
            m = re.match(r"\s*\w+(?:\[(\d+)\])?\s*$", name)
            total += TYPE_BYTES[typ] * (int(m.group(1)) if m.group(1) else 1)
    return total


def test_registry_has_27_profiles_plus_nvfp4():
    assert len(GGUF) == 27
    assert set(ALL) == set(GGUF) | {"nvfp4"}


@pytest.mark.parametrize("fmt", GGUF)
def test_block_bytes_equal_layout_field_sum(fmt):
    _, B, S, T = oracle.info(fmt)
    assert S == _field_bytes(LAYOUT_FIELDS[fmt[5:]])
    assert T == 0


@pytest.mark.parametrize("name", sorted(NINFER_GGUF))
def test_block_geometry_matches_ninfer_table(name):
    _, B, S, _ = oracle.info("gguf:" + name)
    b_ref, s_ref, bpw = NINFER_GGUF[name]
    assert (B, S) == (b_ref, s_ref)
    assert 8 * S / B == bpw


def test_nvfp4_divisor_variant_geometry():
    # gguf:nvfp4 block bytes (64 values, 36 bytes) plus one 4-byte divisor
    assert oracle.info("nvfp4")[1:] == (64, 36, 4)
    assert oracle.info("gguf:nvfp4")[1:] == (64, 36, 0)


# --------------------------------------------------------------------------
# Length rule: "Format identifiers" (closed form) and the Kiln quantization
# page's scale-count formula ceil(shape[axis]/group) * prod(other dims).
# --------------------------------------------------------------------------
def _kiln_count(shape, group):
    others = 1  # the product of no dimensions is 1
    for d in shape[:-1]:
        others *= d
    return -(-shape[-1] // group) * others


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("shape", [[32 * 256], [3, 512], [2, 3, 1024], [7, 256]])
def test_length_rule_closed_form(fmt, shape):
    _, B, S, T = oracle.info(fmt)
    st, nb, ne = oracle.sizes(fmt, shape)
    assert st == oracle.OK
    assert ne == int(np.prod(shape))
    assert nb == _kiln_count(shape, B) * S + T


def test_kiln_examples():
    # a rank-1 tensor of 32 elements with group 32 needs one scale: one MXFP4 block
    st, nb, ne = oracle.sizes("gguf:mxfp4", [32])
    assert (st, nb, ne) == (oracle.OK, 17, 32)
    assert _kiln_count([32], 32) == 1


@pytest.mark.parametrize("shape,status", [
    ([], oracle.ERR_RANK), ([-1, 32], oracle.ERR_DIM), ([4, 31], oracle.ERR_ALIGN),
    ([0, 33], oracle.ERR_ALIGN), ([2 ** 40, 2 ** 40, 32], oracle.ERR_OVERFLOW),
])
def test_length_rule_rejections(shape, status):
    assert oracle.sizes("gguf:q4_0", shape)[0] == status


def test_empty_tensors():
    assert oracle.sizes("gguf:q4_k", [0, 256]) == (oracle.OK, 0, 0)
    assert oracle.sizes("gguf:q4_k", [5, 0]) == (oracle.OK, 0, 0)
    assert oracle.sizes("nvfp4", [0, 64]) == (oracle.OK, 4, 0)
    # a zero anywhere makes the count exactly zero, however large the rest
    assert oracle.sizes("gguf:q4_0", [2 ** 62, 0, 32])[0] == oracle.OK


@pytest.mark.parametrize("delta", [-36, -1, 1, 36])
def test_wrong_length_rejected(delta):
    p = synth.payload("gguf:q8_1", 8, 1, RECIPE)
    bad = np.zeros(p.size + delta, dtype=np.uint8) if delta > 0 else p[:delta]
    assert oracle.decode_status("gguf:q8_1", bad, [8 * 32]) == oracle.ERR_LENGTH


# --------------------------------------------------------------------------
# Word conversions versus library routines.
# --------------------------------------------------------------------------
def test_binary16_all_words_match_numpy():
    words = np.arange(65536, dtype=np.uint16)
    ref = words.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(w)) for w in words], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _structured_f32_sample():
    """Every high half (sign, exponent, top mantissa bits) with low halves at
    and around the rounding points of both bf16 and f16 (f16's odd-LSB ties,
    and the tie points one and two bits up that its subnormal range moves
    them to), plus random words."""
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x2FFF, 0x3000,
                     0x3001, 0x3FFF, 0x4000, 0x4001, 0x5FFF, 0x6000, 0x6001, 0x7FFF, 0x8000, 0x8001,
                     0xBFFF, 0xC000, 0xC001, 0xFFFF], dtype=np.uint32)
    words = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(2024)
    rand = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([words, rand]).view(np.float32)


def test_bf16_rne_matches_torch():
    x = _structured_f32_sample()
    got = oracle.convert(x, "bf16")
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN with its sign
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)
    assert np.array_equal(got[nan] >> 15, (x[nan].view(np.uint32) >> 31).astype(np.uint16))


def test_f16_rne_matches_numpy():
    x = _structured_f32_sample()
    got = oracle.convert(x, "f16")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f16_rne_overflow_and_subnormal_edges():
    cases = {65504.0: 0x7BFF, 65519.99: 0x7BFF, 65520.0: 0x7C00, 2.0 ** -24: 0x0001,
             2.0 ** -25: 0x0000, 1.5 * 2.0 ** -25: 0x0001, 3 * 2.0 ** -25: 0x0002,
             2.0 ** -14: 0x0400, -0.0: 0x8000}
    for v, bits in cases.items():
        assert int(oracle.convert(np.array([v], np.float32), "f16")[0]) == bits, v


def test_e4m3fn_all_words_match_torch():
    words = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = words.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3fn_to_f32(w) for w in range(256)], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_output_types_match_libraries():
    for fmt in ("gguf:q4_k", "gguf:iq2_xxs", "gguf:mxfp4", "nvfp4", "gguf:q8_k"):
        _, B, S, T = oracle.info(fmt)
        p = synth.payload(fmt, 64, 11, synth.raw() if fmt != "nvfp4" else RECIPE)
        shape = [64 * B]
        f32 = oracle.decode(fmt, p, shape, "f32")
        nan = np.isnan(f32)
        bf = oracle.decode(fmt, p, shape, "bf16")
        ref_bf = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(bf[~nan], ref_bf[~nan])
        with np.errstate(over="ignore"):
            ref_h = f32.astype(np.float16).view(np.uint16)
        assert np.array_equal(oracle.decode(fmt, p, shape, "f16")[~nan], ref_h[~nan])
        f64 = oracle.decode(fmt, p, shape, "f64")
        assert np.array_equal(f64[~nan], f32[~nan].astype(np.float64))
        assert np.array_equal(np.isnan(f64), nan)


# --------------------------------------------------------------------------
# Scale decodes: closed forms and library routines.
# --------------------------------------------------------------------------
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # NInfer page 3.3, positive code words


def test_mxfp4_every_exponent_byte_and_code():
    """Half scale x doubled E2M1 equals the OCP MX value 2^(e-127) * E2M1(code);
    both zeros are +0; e = 255 keeps the page's 2^127 half scale."""
    blocks = []
    for e in range(256):
        blocks.append(bytes([e]) + bytes([c | (c << 4) for c in range(16)]))
    y = oracle.decode_blocks_f32("gguf:mxfp4", np.frombuffer(b"".join(blocks), np.uint8))
    y = y.reshape(256, 32)
    for e in range(256):
        for code in range(16):
            mag = E2M1[code & 7]
            sign = -1.0 if (code & 8) and mag != 0 else 1.0
            with np.errstate(over="ignore"):
                ref = np.float32(sign * math.ldexp(mag, e - 127)) if e < 255 else \
                    np.float32(sign * mag * 2.0 * 2.0 ** 127)
            for j in (code, 16 + code):
                assert y[e, j].view(np.uint32) == np.array(ref).view(np.uint32), (e, code)
    # e = 127: the plain E2M1 values (scale 1.0)
    assert list(y[127, :8]) == E2M1


def test_gguf_nvfp4_every_scale_byte_and_code():
    """Half scale = unsigned E4M3 value / 2 with bit 7 ignored, computed with
    PyTorch's float8_e4m3fn on the low 7 bits; the whole byte 127 gives 0 and
    0xFF (E=15, m=7 once bit 7 is dropped) gives 240."""
    low7 = torch.arange(128, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ue4m3 = low7.to(torch.float32).numpy()
    blocks = []
    for e in range(256):
        blocks.append(bytes([e, 0x38, 0x38, 0x38]) + bytes([c | (c << 4) for c in range(8)] +
                                                           [(c + 8) | ((c + 8) << 4) for c in range(8)]) +
                      bytes(16))
    y = oracle.decode_blocks_f32("gguf:nvfp4", np.frombuffer(b"".join(blocks), np.uint8)).reshape(256, 64)
    V = [0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12]
    for e in range(256):
        if e == 127:
            half = 0.0
        elif (e & 0x7F) == 0x7F:
            half = 240.0
        else:
            half = float(ue4m3[e & 0x7F]) / 2
        for j in range(8):
            assert y[e, j] == np.float32(half * V[j]), (e, j)
            assert y[e, 8 + j] == np.float32(half * V[j]), (e, j)
    # spot values of the scale byte
    assert y[0x38, 1] == 0.5 and y[0x7E, 2] == 448.0 and y[0x01, 2] == 2.0 ** -9
    assert y[0x80, 2] == 0.0 and y[0xFF, 2] == 480.0


# --------------------------------------------------------------------------
# Q8 family: y = d*q in binary32 (numpy's IEEE multiply); cached fields ignored.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,doff,qoff,n,dbytes", [
    ("gguf:q8_0", 0, 2, 32, 2), ("gguf:q8_1", 0, 4, 32, 2), ("gguf:q8_k", 0, 4, 256, 4)])
def test_q8_is_d_times_q(fmt, doff, qoff, n, dbytes):
    _, B, S, _ = oracle.info(fmt)
    p = synth.payload(fmt, 200, 5, synth.raw())
    y = oracle.decode(fmt, p, [200 * B]).reshape(200, B)
    blk = p.reshape(200, S)
    dt = np.float16 if dbytes == 2 else np.float32
    d = blk[:, doff:doff + dbytes].copy().view(dt).astype(np.float32)
    q = blk[:, qoff:qoff + n].view(np.int8).astype(np.float32)
    ref = d * q
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert np.array_equal(y[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("fmt,start,stop", [("gguf:q8_1", 2, 4), ("gguf:q8_k", 260, 292)])
def test_q8_cached_sums_ignored(fmt, start, stop):
    _, B, S, _ = oracle.info(fmt)
    p = synth.payload(fmt, 16, 9, RECIPE)
    y0 = oracle.decode(fmt, p, [16 * B])
    rng = np.random.default_rng(0)
    for t in range(start, stop):
        q = p.copy()
        q.reshape(16, S)[:, t] ^= rng.integers(1, 256, size=16).astype(np.uint8)
        assert np.array_equal(oracle.decode(fmt, q, [16 * B]).view(np.uint32), y0.view(np.uint32))


def test_q1_0_is_plus_minus_d():
    p = synth.payload("gguf:q1_0", 50, 3, synth.raw())
    y = oracle.decode("gguf:q1_0", p, [50 * 128]).reshape(50, 128)
    blk = p.reshape(50, 18)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float32)[:, 0]
    bits = np.unpackbits(blk[:, 2:], axis=1, bitorder="little")
    ref = np.where(bits == 1, d[:, None], -d[:, None])
    nan = np.isnan(ref)
    assert np.array_equal(y[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --------------------------------------------------------------------------
# nvfp4 with divisor (NInfer page 3.3): the exact product e2m1 * e4m3fn is
# divided once; numpy computes the quotient in binary64 and rounds to
# binary32 (double rounding is innocuous for division at 53 >= 2*24+2 bits).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d_w", [1.0, 3.0, 448.0, 7.1234567, 1e-30, 3.4e38])
def test_nvfp4_divisor_against_binary64(d_w):
    scales = list(range(0x00, 0x7F))  # every valid (sign-zero, finite) scale word
    e4 = torch.tensor(scales, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    e4 = e4.to(torch.float64).numpy()
    blocks = b""
    for s in scales:
        blocks += bytes([s, s, s, s]) + bytes([c | ((c ^ 8) << 4) for c in range(8)] * 4)
    n = len(scales)
    payload = np.frombuffer(blocks + np.array([d_w], "<f4").tobytes(), np.uint8)
    y = oracle.decode("nvfp4", payload, [n * 64]).reshape(n, 64)
    dw = float(np.float32(d_w))
    for bi in range(n):
        for j in range(16):
            code = j if j < 8 else (j - 8) ^ 8
            mag = E2M1[code & 7]
            e2 = -mag if code & 8 else mag
            ref = np.float32(np.float64(e2) * e4[bi] / np.float64(dw))
            assert y[bi, j].view(np.uint32) == np.array(ref).view(np.uint32), (bi, j)


# --------------------------------------------------------------------------
# Codebooks: "IQ codebooks" row counts, value ranges, distinct rows.
# --------------------------------------------------------------------------
ROWS = {"iq2xxs_grid": (256, 8), "iq2xs_grid": (512, 8), "iq2s_grid": (1024, 8),
        "iq3xxs_grid": (256, 4), "iq3s_grid": (512, 4), "iq1s_grid": (2048, 8)}
VALUES = {"iq2xxs_grid": {8, 25, 43}, "iq2xs_grid": {8, 25, 43}, "iq2s_grid": {8, 25, 43},
          "iq3xxs_grid": {4, 12, 20, 28, 36, 44, 52, 62}, "iq3s_grid": {1, 3, 5, 7, 9, 11, 13, 15},
          "iq1s_grid": {-1, 0, 1}}


@pytest.mark.parametrize("book", sorted(ROWS))
def test_codebook_shape_and_distinct_rows(book):
    g = oracle.grid(book)
    assert g.shape == ROWS[book]
    assert set(np.unique(g)) <= VALUES[book]
    assert len({tuple(r) for r in g}) == g.shape[0]


def test_codebook_fields_in_range_and_spot_rows():
    assert oracle.grid_bad_fields() == 0
    assert list(oracle.grid("iq2xxs_grid")[0]) == [8] * 8
    assert list(oracle.grid("iq1s_grid")[0]) == [-1] * 8
    assert list(oracle.grid("iq1s_grid")[2047]) == [1] * 8
    assert list(oracle.grid("iq3s_grid")[0]) == [1] * 4
    assert list(oracle.grid("iq3xxs_grid")[0]) == [4] * 4


# --------------------------------------------------------------------------
# Hand-derived one-block examples (tests/golden/one_block.json).
# --------------------------------------------------------------------------
def _golden():
    with open(os.path.join(HERE, "golden", "one_block.json")) as f:
        return json.load(f)["examples"]


def _expand(runs, n, bits32=True):
    out = np.zeros(n, dtype=np.uint32 if bits32 else np.uint16)
    seen = np.zeros(n, dtype=bool)
    for lo, hi, v in runs:
        if isinstance(v, str):
            w = int(v, 16)
        else:
            w = int(np.array([v], np.float32).view(np.uint32)[0])
        out[lo:hi + 1] = w
        seen[lo:hi + 1] = True
    assert seen.all()
    return out


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["id"])
def test_golden_one_block(ex):
    fmt = ex["format"]
    _, B, S, T = oracle.info(fmt)
    p = np.frombuffer(bytes.fromhex(ex["payload"]), np.uint8)
    y = oracle.decode(fmt, p, [B], "f32")
    assert np.array_equal(y.view(np.uint32), _expand(ex["expect"], B))
    if "expect_bf16" in ex:
        yb = oracle.decode(fmt, p, [B], "bf16")
        assert np.array_equal(yb, _expand(ex["expect_bf16"], B, bits32=False))


# --------------------------------------------------------------------------
# Second reading: the page's own Python notation, on random corpora.
# --------------------------------------------------------------------------
NOTATION = page_notation.load()


@pytest.mark.skipif(NOTATION is None, reason="NQ_PAGE_TEXT does not name a copy of the page text")
@pytest.mark.parametrize("fmt", GGUF)
@pytest.mark.parametrize("recipe", [synth.raw(), RECIPE], ids=repr)
def test_oracle_matches_page_python_notation(fmt, recipe):
    _, B, S, _ = oracle.info(fmt)
    nb = 24
    p = synth.payload(fmt, nb, 77, recipe)
    y = oracle.decode(fmt, p, [nb * B])
    ref = []
    for i in range(nb):
        ref += NOTATION["decode_block"](list(bytes(p[i * S:(i + 1) * S])), page_notation.kind_of(fmt))
    ref = np.array(ref, dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert np.array_equal(y[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.skipif(NOTATION is None, reason="NQ_PAGE_TEXT does not name a copy of the page text")
def test_oracle_codebooks_match_page_python_notation():
    for book in ROWS:
        g = oracle.grid(book)
        for r in range(g.shape[0]):
            assert list(g[r]) == NOTATION["grid"](book, r)


# --------------------------------------------------------------------------
# Structure: flipping one payload bit changes only the outputs the layout
# table and the element-order rules say it can reach.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ALL)
def test_bit_flip_structure(fmt):
    _, B, S, T = oracle.info(fmt)
    m = layout_map.build(fmt)
    trials = 6
    base = synth.payload(fmt, trials, 1234, RECIPE)
    d_w = 3.0
    blocks = base[:trials * S]
    y0 = oracle.decode_blocks_f32(fmt, blocks, d_w).reshape(trials, B).view(np.uint32)
    for key, (kind, outs) in m.m.items():
        byte, bit = divmod(key, 8)
        flipped = blocks.copy().reshape(trials, S)
        flipped[:, byte] ^= np.uint8(1 << bit)
        y1 = oracle.decode_blocks_f32(fmt, flipped.ravel(), d_w).reshape(trials, B).view(np.uint32)
        union = set()
        for t in range(trials):
            changed = set(np.nonzero(y0[t] != y1[t])[0].tolist())
            assert changed <= outs, (fmt, byte, bit, sorted(changed - outs)[:8])
            union |= changed
        if kind == "exact":
            assert union == set(outs), (fmt, byte, bit, sorted(set(outs) - union)[:8])
        elif kind == "some":
            assert union, (fmt, byte, bit)


# ---------------------------------------------------------------------------
# nvfp4 with stacked divisors (NInfer tensor-formats, section 3.3: one weight
# divisor per source matrix stacked into the plane, covering N / divisors
# consecutive rows in stacking order).
# ---------------------------------------------------------------------------
def _stacked(shape, divisors, seed, d_ws=None):
    K = shape[-1]
    N = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    nb = N * K // 64
    return synth.payload("nvfp4", nb, seed, synth.binade(-12, -6, True), divisor=d_ws, divisors=divisors), N, K


@pytest.mark.parametrize("shape,divisors", [([12, 128], 1), ([12, 128], 2), ([12, 128], 3), ([12, 128], 4),
                                            ([12, 128], 12), ([2, 6, 64], 3), ([8, 256], 2)])
def test_nvfp4_stacked_equals_each_source_decoded_alone(shape, divisors):
    """A stacked plane decodes as its sources would one by one: source j is the
    rows [j N/D, (j+1) N/D) with the j-th trailer word as its only divisor."""
    p, N, K = _stacked(shape, divisors, 101 + divisors)
    got = oracle.decode_nvfp4_stacked(p, shape, divisors, "f32").view(np.uint32)
    rows = N // divisors
    src_bytes = rows * (K // 64) * 36
    trailer = p[N * (K // 64) * 36:]
    for j in range(divisors):
        alone = np.concatenate([p[j * src_bytes:(j + 1) * src_bytes], trailer[4 * j:4 * j + 4]])
        ref = oracle.decode("nvfp4", alone, [rows, K], "f32").view(np.uint32)
        assert np.array_equal(got[j * rows * K:(j + 1) * rows * K], ref), j


def test_nvfp4_stacked_power_of_two_divisors_scale_exactly():
    """Every source holds the same blocks and d_w[j] = 2^j, so source j is
    source 0 divided by 2^j exactly (all values stay normal binary32)."""
    K, rows, D = 128, 3, 4
    one = synth.payload("nvfp4", rows * K // 64, 7, synth.binade(-12, -6, True), divisor=1.0)[:-4]
    p = np.concatenate([np.tile(one, D), np.array([2.0 ** j for j in range(D)], dtype="<f4").view(np.uint8)])
    y = oracle.decode_nvfp4_stacked(p, [D * rows, K], D, "f64").reshape(D, rows * K)
    assert np.any(y[0] != 0)
    for j in range(D):
        assert np.array_equal(y[j], y[0] / 2.0 ** j)
    # the trailer length tells the stacking apart: one divisor means 12 bytes fewer
    assert oracle.sizes_nvfp4_stacked([D * rows, K], 1)[1] == p.size - 12


def test_nvfp4_stacked_single_divisor_is_plain_nvfp4():
    p, N, K = _stacked([5, 192], 1, 33)
    for dtype in ("f32", "bf16", "f16", "f64"):
        assert np.array_equal(oracle.decode_nvfp4_stacked(p, [5, 192], 1, dtype),
                              oracle.decode("nvfp4", p, [5, 192], dtype))


@pytest.mark.parametrize("shape,divisors,want", [
    ([12, 128], 0, "ERR_DIVISORS"), ([12, 128], -3, "ERR_DIVISORS"), ([12, 128], 5, "ERR_DIVISORS"),
    ([12, 128], 6, "OK"), ([6, 0], 4, "ERR_DIVISORS"), ([6, 0], 3, "OK"), ([0, 128], 7, "OK"),
    ([128], 1, "OK"), ([128], 2, "ERR_DIVISORS"), ([12, 100], 2, "ERR_ALIGN"), ([3, 4, 64], 4, "OK"),
    ([3, 4, 64], 8, "ERR_DIVISORS"), ([2 ** 40, 2 ** 40, 0], 1, "ERR_OVERFLOW")])
def test_nvfp4_stacked_length_rule(shape, divisors, want):
    """nbytes = prod(shape[:-1]) (shape[-1]/64) 36 + 4 divisors, with
    N = prod(shape[:-1]) a multiple of divisors (the product of no dimensions
    is 1)."""
    st, nbytes, nelems = oracle.sizes_nvfp4_stacked(shape, divisors)
    assert st == getattr(oracle, want), (st, want)
    if st == oracle.OK:
        N = math.prod(shape[:-1])
        assert nbytes == N * (shape[-1] // 64) * 36 + 4 * divisors
        assert nelems == N * shape[-1]
        p = np.zeros(nbytes, dtype=np.uint8)
        assert len(oracle.decode_nvfp4_stacked(p, shape, divisors)) == nelems
        with pytest.raises(ValueError):
            oracle.decode_nvfp4_stacked(np.zeros(nbytes + 1, dtype=np.uint8), shape, divisors)


# ---------------------------------------------------------------------------
# Row-scaled FP8 (NInfer tensor-formats, section 3.3): w_hat = binary32(c32 * s32).
# ---------------------------------------------------------------------------
def test_bf16_words_against_torch():
    """Every bfloat16 word against torch's conversion (NaN by class)."""
    w = np.arange(1 << 16, dtype=np.uint32)
    ref = torch.from_numpy(w.astype(np.int32)).to(torch.int16).view(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.bf16_to_f32(int(x)) for x in w], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(got[nan]), np.signbit(ref[nan]))


def _fp8_payload(codes, scale_words):
    return np.concatenate([np.asarray(codes, np.uint8).ravel(), np.asarray(scale_words, "<u2").view(np.uint8)])


@pytest.mark.parametrize("fmt", ["fp8_e4m3fn_row_bf16", "fp8_e4m3fn_row_fp16"])
def test_fp8_row_every_code_against_binary64(fmt):
    """All 256 codes times scale words of every class: each value is the
    binary64 product (exact: at most 4 x 11 significant bits) rounded once to
    binary32, as torch computes it from its own float8/bfloat16/float16."""
    scales = ([0x3F80, 0x4000, 0x0001, 0x007F, 0x0080, 0x7F7F, 0x7F80, 0xFF80, 0x8000, 0x0000, 0x7FC1, 0xC2F7, 0x3E2B]
              if fmt.endswith("bf16") else
              [0x3C00, 0x4000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x7C00, 0xFC00, 0x8000, 0x0000, 0x7E01, 0xC8F7, 0x3555])
    N, K = len(scales), 256
    codes = np.tile(np.arange(256, dtype=np.uint8), (N, 1))
    y = oracle.decode_fp8_row(fmt, _fp8_payload(codes, scales), [N, K], "f32").reshape(N, K)
    c64 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sdt = torch.bfloat16 if fmt.endswith("bf16") else torch.float16
    s64 = torch.tensor(scales, dtype=torch.int32).to(torch.int16).view(sdt).to(torch.float64).numpy()
    with np.errstate(invalid="ignore", over="ignore"):
        ref = (s64[:, None] * c64[None, :]).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert np.array_equal(y[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_fp8_row_golden_examples():
    path = os.path.join(os.path.dirname(__file__), "golden", "fp8_row.json")
    for ex in json.load(open(path))["examples"]:
        p = np.frombuffer(bytes.fromhex(ex["payload"]), np.uint8)
        y = oracle.decode_fp8_row(ex["format"], p, ex["shape"], "f32")
        assert y.size == len(ex["expect"]), ex["id"]
        for v, want in zip(y, ex["expect"]):
            if want == "nan":
                assert np.isnan(v), ex["id"]
            elif isinstance(want, str):
                assert int(np.array(v, np.float32).view(np.uint32)) == int(want, 16), (ex["id"], v, want)
            else:
                assert np.array(v, np.float32).view(np.uint32) == np.array(want, np.float32).view(np.uint32), \
                    (ex["id"], v, want)


def test_fp8_row_structure():
    """A code word changes only its own output; a scale word only its row."""
    N, K = 5, 37
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x11  # keep NaN words out
    scales = np.array([0x3F80, 0x4040, 0x3E00, 0x4300, 0x3C23], np.uint16)
    base = oracle.decode_fp8_row("fp8_e4m3fn_row_bf16", _fp8_payload(codes, scales), [N, K], "f32").reshape(N, K)
    for (n, k) in [(0, 0), (2, 17), (4, 36)]:
        c2 = codes.copy()
        c2[n, k] ^= 0x41
        y = oracle.decode_fp8_row("fp8_e4m3fn_row_bf16", _fp8_payload(c2, scales), [N, K], "f32").reshape(N, K)
        diff = np.argwhere(y.view(np.uint32) != base.view(np.uint32))
        assert [tuple(d) for d in diff] == [(n, k)]
    for n in range(N):
        s2 = scales.copy()
        s2[n] ^= 0x0080
        y = oracle.decode_fp8_row("fp8_e4m3fn_row_bf16", _fp8_payload(codes, s2), [N, K], "f32").reshape(N, K)
        rows = set(np.argwhere(y.view(np.uint32) != base.view(np.uint32))[:, 0])
        assert rows == {n}


@pytest.mark.parametrize("shape,want", [([3, 5], "OK"), ([1, 1], "OK"), ([0, 5], "ERR_DIM"), ([3, 0], "ERR_DIM"),
                                        ([-1, 5], "ERR_DIM"), ([15], "ERR_RANK"), ([1, 3, 5], "ERR_RANK"),
                                        ([], "ERR_RANK"), ([2 ** 62, 4], "ERR_OVERFLOW"),
                                        ([2 ** 31, 2 ** 31], "ERR_OVERFLOW")])
def test_fp8_row_length_rule(shape, want):
    """Rank two, positive dimensions, nbytes = N*K + 2N (and N*K*8 within INT64)."""
    st, nbytes, nelems = oracle.sizes_fp8_row(shape)
    assert st == getattr(oracle, want), st
    if st == oracle.OK:
        assert nbytes == shape[0] * shape[1] + 2 * shape[0] and nelems == shape[0] * shape[1]
        with pytest.raises(ValueError):
            oracle.decode_fp8_row("fp8_e4m3fn_row_bf16", np.zeros(nbytes - 1, np.uint8), shape)


# ---------------------------------------------------------------------------
# grouped_absmax encoder (NInfer tensor-formats, section 7.2).
# ---------------------------------------------------------------------------
def _f32(v):
    if isinstance(v, str):
        return np.array([int(v, 16)], np.uint32).view(np.float32)[0]
    return np.float32(v)


def test_grouped_absmax_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "grouped_absmax.json")
    for ex in json.load(open(path))["examples"]:
        x = np.array([[_f32(v) for v in ex["x"]]], np.float32)
        st, codes, scales = oracle.grouped_absmax(ex["scheme"], x)
        assert st == ex["status"], ex["id"]
        if st == 0:
            assert list(codes[0]) == ex["codes"], (ex["id"], list(codes[0]))
            assert [hex(s) for s in scales[0]] == [hex(int(s, 16)) for s in ex["scales"]], ex["id"]


@pytest.mark.parametrize("scheme", sorted(oracle.GQ_SCHEMES))
def test_grouped_absmax_invariants(scheme):
    """On random rows (log-uniform magnitudes, random signs, zero groups,
    partial last groups): codes lie in [qmin, qmax]; each scale is the
    binary16 rounding of amax / qmax (or the rescue, or +0 for a zero group);
    a code that is not clamped reconstructs its value within half a scale
    step; with a normal binary16 scale the largest magnitude maps to +-qmax
    or qmin; zero groups are zero."""
    sid, G, qmin, qmax = oracle.GQ_SCHEMES[scheme]
    rng = np.random.default_rng(sid)
    N, K = 9, 3 * G + 5
    x = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-34, 12, (N, 1)))).astype(np.float32)
    x[2, :G] = 0.0
    x[3, G:2 * G] = -0.0
    st, codes, scales = oracle.grouped_absmax(scheme, x)
    assert st == 0
    assert codes.min() >= qmin and codes.max() <= qmax
    s32 = torch.from_numpy(scales.astype(np.int32)).to(torch.int16).view(torch.float16).to(torch.float64).numpy()
    for n in range(N):
        for g in range((K + G - 1) // G):
            v = x[n, g * G:(g + 1) * G].astype(np.float64)
            q = codes[n, g * G:(g + 1) * G].astype(np.float64)
            amax = np.abs(v).max()
            if amax == 0:
                assert scales[n, g] == 0 and not q.any()
                continue
            want = np.float64(np.float16(np.float32(amax / qmax)))  # binary16 RNE of the binary32 quotient
            assert s32[n, g] == (want if want > 0 else 2.0 ** -24)
            inner = (q > qmin) & (q < qmax)
            assert np.all(np.abs(v[inner] - s32[n, g] * q[inner]) <= 0.5 * s32[n, g] * (1 + 2.0 ** -20))
            if s32[n, g] >= 2.0 ** -14:  # a normal binary16 scale is within 2^-11 of amax / qmax
                top = np.argmax(np.abs(v))
                assert q[top] in (qmax, qmin, -qmax) and np.sign(q[top]) == np.sign(v[top])


def test_grouped_absmax_source_types():
    """binary16, bfloat16 and binary64 sources encode as their binary32 values
    (torch converts them independently); a binary64 value past binary32
    fails as non-finite."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((4, 70)) * 3).astype(np.float32)
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        t = torch.from_numpy(x).to(tdt)
        words = t.view(torch.int16).numpy().view(np.uint16)
        want = oracle.grouped_absmax("q5_g64_fp16", t.to(torch.float32).numpy())
        got = oracle.grouped_absmax("q5_g64_fp16", words, dt)
        assert got[0] == 0 and np.array_equal(got[1], want[1]) and np.array_equal(got[2], want[2])
    x64 = x.astype(np.float64) * (1 + 1e-9)
    want = oracle.grouped_absmax("q8_g32_fp16", x64.astype(np.float32))
    got = oracle.grouped_absmax("q8_g32_fp16", x64, "f64")
    assert np.array_equal(got[1], want[1]) and np.array_equal(got[2], want[2])
    assert oracle.grouped_absmax("q8_g32_fp16", np.array([[1e39, 1.0]]), "f64")[0] == 1


def test_grouped_absmax_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.grouped_absmax("q4_g64_fp16", np.zeros((0, 64), np.float32))
    with pytest.raises(ValueError):
        oracle.grouped_absmax("q4_g64_fp16", np.zeros((3, 0), np.float32))
