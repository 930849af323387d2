"""Pins of the oracle's linear product with q8_1 activations (CPU only).

What is pinned, and against what:
  * the activation quantizer: hand-derived blocks (tests/golden/q8_1_activation.json);
    the pinned q8_g32_fp16 encoder and the pinned gguf:q8_1 decoder (the block's
    codes, d and represented values); numpy's binary16 rounding for the sum field;
  * the product: numpy's float64 matmul of the pinned decoders' outputs, on
    non-square shapes for every gguf format; a hand-built example;
  * the criterion's scale env: |w| * |x| summed (numpy) for formats whose value
    is a scale times a code; for the five formats with a code-independent term,
    that the term is constant over each sub-block and equals the value at code 0
    (the zeroed bytes hold exactly the code bits);
  * the criterion itself: float32 evaluations in several orders stay inside it.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from linear_criterion import criterion

HERE = os.path.dirname(os.path.abspath(__file__))
GGUF = [f for f in oracle.format_names() if f.startswith("gguf:")]
AFFINE = {"gguf:q4_1": 32, "gguf:q5_1": 32, "gguf:q2_k": 16, "gguf:q4_k": 32, "gguf:q5_k": 32}
CODE_BITS = {"gguf:q4_1": 4, "gguf:q5_1": 5, "gguf:q2_k": 2, "gguf:q4_k": 4, "gguf:q5_k": 5}


def _golden():
    with open(os.path.join(HERE, "golden", "q8_1_activation.json")) as f:
        return json.load(f)["cases"]


def _expand(d, fill=0.0):
    out = np.full(32, fill, dtype=np.float64)
    for k, v in d.items():
        if k == "all":
            out[:] = v
        else:
            out[int(k)] = float("nan") if v == "nan" else v
    return out


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["id"])
def test_q8_1_golden(case):
    x = _expand(case["x"]).astype(np.float32)[None, :]
    st, blocks = oracle.quantize_q8_1(x)
    assert st == case["status"]
    if st & 3:
        return  # a failed block is unspecified
    b = blocks[0, 0]
    assert int(b[0]) | int(b[1]) << 8 == int(case["d16"], 16)
    assert int(b[2]) | int(b[3]) << 8 == int(case["s16"], 16)
    codes = _expand(case["codes"]).astype(np.int64)
    assert np.array_equal(b[4:].view(np.int8).astype(np.int64), codes)


def _act(M, K, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * scale
    x[:, rng.integers(0, K, size=max(1, K // 97))] *= 25.0  # outlier columns
    return x


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
def test_q8_1_matches_grouped_encoder_and_decoder(in_dtype):
    """Codes and d are the q8_g32_fp16 encoder's; the gguf:q8_1 decoder of the
    blocks gives d32 * code; the sum field is binary16(d32 * sum of codes)."""
    M, K = 3, 352
    x = _act(M, K, 11)
    if in_dtype == "f32":
        xs = x.astype(np.float32)
    elif in_dtype == "f16":
        xs = x.astype(np.float16).view(np.uint16)
    else:
        xs = oracle.convert(x.astype(np.float32), "bf16").reshape(M, K)
    st, blocks = oracle.quantize_q8_1(xs, in_dtype)
    assert st == 0
    gst, codes, scales = oracle.grouped_absmax("q8_g32_fp16", xs, in_dtype)
    assert gst == 0
    q = blocks[:, :, 4:].view(np.int8).reshape(M, K)
    assert np.array_equal(q, codes)
    d16 = blocks[:, :, 0].astype(np.uint16) | blocks[:, :, 1].astype(np.uint16) << 8
    assert np.array_equal(d16, scales)
    s16 = blocks[:, :, 2].astype(np.uint16) | blocks[:, :, 3].astype(np.uint16) << 8
    d = d16.view(np.float16).astype(np.float64)
    want = (d * q.reshape(M, K // 32, 32).astype(np.int64).sum(-1)).astype(np.float16).view(np.uint16)
    assert np.array_equal(s16, want)
    xh = oracle.decode("gguf:q8_1", blocks.reshape(-1), [M, K])
    assert np.array_equal(xh.reshape(M, K), (np.repeat(d, 32, axis=1) * q).astype(np.float32))


def test_q8_1_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize_q8_1(np.zeros((2, 48), np.float32))


def _weights(fmt, N, K, seed):
    _, B, S, _ = oracle.info(fmt)
    rec = synth.binade(-6, -2, fmt in ("gguf:q4_0", "gguf:q8_0", "gguf:q5_0", "gguf:iq4_nl"))
    return synth.payload(fmt, N * K // B, seed, rec)


def _shape(fmt):
    B = oracle.info(fmt)[1]
    return 5, 2 * max(B, 128)


@pytest.mark.parametrize("fmt", GGUF)
def test_gemv_matches_numpy(fmt):
    """y = x_hat @ w_hat^T (numpy float64) from the pinned decoders; env is
    sum |w| |x| for the scale-times-code formats."""
    N, K = _shape(fmt)
    M = 3
    w = _weights(fmt, N, K, 1234)
    _, xq = oracle.quantize_q8_1(_act(M, K, 5).astype(np.float32))
    y, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    wh = oracle.decode(fmt, w, [N, K]).astype(np.float64).reshape(N, K)
    xh = oracle.decode("gguf:q8_1", xq.reshape(-1), [M, K]).astype(np.float64).reshape(M, K)
    ref = xh @ wh.T
    mag = np.abs(xh) @ np.abs(wh).T
    assert np.all(np.abs(y - ref) <= 4 * K * 2.0 ** -53 * mag)
    if fmt in AFFINE:
        assert np.all(env >= mag * (1 - 1e-12))
    else:
        assert np.allclose(env, mag, rtol=4 * K * 2.0 ** -53, atol=0)


def test_gemv_hand_example():
    """Two q8_0 rows of one block: row 0 d = 1, codes 0..31; row 1 d = 0.5,
    codes -1.  The activation is 127 at k = 5 (d = 1, code 127): y = 5*127 and
    -0.5*127."""
    blk = np.zeros((2, 34), np.uint8)
    blk[0, :2] = [0x00, 0x3C]
    blk[0, 2:] = np.arange(32, dtype=np.int8).view(np.uint8)
    blk[1, :2] = [0x00, 0x38]
    blk[1, 2:] = np.full(32, -1, np.int8).view(np.uint8)
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = 127
    _, xq = oracle.quantize_q8_1(x)
    y, env = oracle.gemv_q8_1("gguf:q8_0", blk.reshape(-1), 2, 32, xq, 1)
    assert y.tolist() == [[635.0, -63.5]]
    assert env.tolist() == [[635.0, 63.5]]


@pytest.mark.parametrize("fmt", sorted(AFFINE))
def test_gemv_offset_term(fmt):
    """For the formats with a code-independent term o, env = sum |x| (|w| + 2|o|)
    where o is the value the weight takes at code 0: over each sub-block o is
    one constant (the zeroed bytes hold every code bit, so no per-weight bit
    survives), w >= o (scales here are positive, codes non-negative), and
    where a weight's code is 0, w == o exactly (o is that value, not merely a
    constant)."""
    N, K = 4, 512
    w = _weights(fmt, N, K, 77)
    wh = oracle.decode(fmt, w, [N, K]).astype(np.float64).reshape(N, K)
    x = np.zeros((K, K), np.float32)
    np.fill_diagonal(x, 127.0)  # activation row k: 127 at k (d = 1, code 127)
    _, xq = oracle.quantize_q8_1(x)
    _, env = oracle.gemv_q8_1(fmt, w, N, K, xq, K)
    o = (env.T / 127.0 - np.abs(wh)) / 2.0  # env[k, n] = 127 (|w| + 2|o|) at weight (n, k): o = |o|
    sub = AFFINE[fmt]
    hits = nonzero = total = 0
    for n in range(N):
        for s0 in range(0, K, sub):
            ws, os_ = wh[n, s0:s0 + sub], o[n, s0:s0 + sub]
            assert np.allclose(os_, os_[0], rtol=1e-14, atol=0)
            total += 1
            nonzero += os_[0] != 0
            hits += np.isclose(abs(ws.min()), os_[0], rtol=1e-14, atol=0)
    assert nonzero > total // 2
    assert hits > total // 2


def test_gemv_errors():
    w = np.zeros(36 * 2 + 4, np.uint8)
    xq = np.zeros(36 * 2, np.uint8)
    with pytest.raises(ValueError):
        oracle.gemv_q8_1("nvfp4", w, 1, 64, xq, 1)
    with pytest.raises(ValueError):  # payload one byte short
        oracle.gemv_q8_1("gguf:q8_0", np.zeros(33, np.uint8), 1, 32, xq[:36], 1)


# --------------------------------------------------------------------------
# The criterion (tests/linear_criterion.py) admits float32 evaluations in
# several orders and rejects a gross mistake.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q6_k", "gguf:q8_0", "gguf:iq2_xxs", "gguf:q4_1"])
def test_criterion_admits_float32_orders(fmt):
    N, K, M = 16, 1024, 2
    w = _weights(fmt, N, K, 9)
    _, xq = oracle.quantize_q8_1(_act(M, K, 2).astype(np.float32))
    y, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    wh = oracle.decode(fmt, w, [N, K]).reshape(N, K).astype(np.float32)
    xh = oracle.decode("gguf:q8_1", xq.reshape(-1), [M, K]).reshape(M, K).astype(np.float32)
    tol = criterion(K, env)
    seq = np.zeros((M, N), np.float32)
    for k in range(K):  # sequential float32 accumulation of rounded products
        seq = (seq + (xh[:, k:k + 1] * wh[None, :, k]).astype(np.float32)).astype(np.float32)
    assert np.all(np.abs(seq.astype(np.float64) - y) <= tol)
    pw = xh @ wh.T  # numpy's float32 matmul (blocked / pairwise)
    assert np.all(np.abs(pw.astype(np.float64) - y) <= tol)
    # per-32 partial sums, then those summed: the shape of a blocked kernel
    part = (xh.reshape(M, 1, K // 32, 32) * wh.reshape(1, N, K // 32, 32)).astype(np.float32).sum(-1,
                                                                                                dtype=np.float32)
    blk = part.sum(-1, dtype=np.float32)
    assert np.all(np.abs(blk.astype(np.float64) - y) <= tol)
    # and a gross mistake does not: drop one 32-value block of every row
    bad = blk - part[:, :, 3]
    assert np.any(np.abs(bad.astype(np.float64) - y) > tol)


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q8_0", "gguf:iq2_xs", "gguf:q2_k", "gguf:tq1_0"])
def test_gemv_matches_numpy_many_rows(fmt):
    """The same product with more activation rows than the single-row kernel
    takes (the batched product's reference)."""
    N, K = _shape(fmt)
    M = 40
    w = _weights(fmt, N, K, 4321)
    _, xq = oracle.quantize_q8_1(_act(M, K, 6).astype(np.float32))
    y, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    wh = oracle.decode(fmt, w, [N, K]).astype(np.float64).reshape(N, K)
    xh = oracle.decode("gguf:q8_1", xq.reshape(-1), [M, K]).astype(np.float64).reshape(M, K)
    ref = xh @ wh.T
    mag = np.abs(xh) @ np.abs(wh).T
    assert np.all(np.abs(y - ref) <= 4 * K * 2.0 ** -53 * mag)
    assert np.all(env >= mag * (1 - 1e-12))
