"""The kernels' own per-thread code, run on the CPU, against the oracle.

The host emulator (tests/emu) executes process<> of nq_kernel.h for every
workgroup and thread, with the launcher's chunk and grid arithmetic, reading
the payload through a source that flags any dword outside the payload.  This
checks indexing, bounds and the decode arithmetic before any GPU run; the
output conversions here are the compiler's software ones, so the GPU tests
remain the authority for the bf16/f16 epilogue.
"""
import numpy as np
import pytest

import block_quantized_weight_nq_amd as nq
import compare
import emu_lib
import oracle
import synth

FORMATS = oracle.format_names()
RAW = synth.raw()
RECIPE = synth.binade(-12, -6, True)


def _oracle(fmt, payload, nblocks, B, dtype):
    return oracle.decode(fmt, payload, [nblocks * B], dtype)


def _same(got, ref, dtype):
    return compare.same(got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_emulated_kernel_matches_oracle(fmt, dtype):
    info = nq.format_query(fmt)
    B = info.block_values
    nblocks = 37
    p = synth.payload(fmt, nblocks, 1000 + info.id, RAW)
    got, bad, msg, guards = emu_lib.decode(info.id, p, nblocks, B, dtype)
    assert bad == 0, msg
    assert guards
    assert _same(got, _oracle(fmt, p, nblocks, B, dtype), dtype)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("mis,out_mis", [(1, 0), (2, 4), (3, 8), (1, 2)])
def test_emulated_misaligned_payload_and_output(fmt, mis, out_mis):
    info = nq.format_query(fmt)
    B = info.block_values
    nblocks = 11
    p = synth.payload(fmt, nblocks, 77, RECIPE)
    dtype = "bf16" if out_mis % 4 else "f32"
    got, bad, msg, guards = emu_lib.decode(info.id, p, nblocks, B, dtype, mis=mis, out_mis=out_mis)
    assert bad == 0, msg
    assert guards
    assert _same(got, _oracle(fmt, p, nblocks, B, dtype), dtype)


def test_emulated_tq1_0_every_byte_at_every_position():
    """tq1_0's base-3 digits: 256 blocks whose byte j is (i + 7 j) mod 256 put
    every byte value (values past 242 included) at every position of a block,
    and so under every digit of the layout; the decode, the single-row product
    and the matrix-core product's span rewrite all take the digits from the
    same rule as the oracle."""
    fmt = "gguf:tq1_0"
    idx, B, S, _ = oracle.info(fmt)
    i = np.arange(256)[:, None]
    j = np.arange(S)[None, :]
    blk = ((i + 7 * j) % 256).astype(np.uint8)
    blk[:, 52:54] = np.array([0x00, 0x3C], np.uint8)  # d = 1.0 keeps every product exact
    p = blk.ravel()
    for dtype in ("f32", "bf16"):
        got, bad, msg, guards = emu_lib.decode(idx, p, 256, B, dtype, mis=1)
        assert bad == 0 and guards, msg
        assert _same(got, _oracle(fmt, p, 256, B, dtype), dtype)
    N, K = 16, 16 * B
    _, xq = oracle.quantize_q8_1(_act(9, K, 3).astype(np.float32))
    for M in (1, 9):
        run = emu_lib.gemv_q8_1 if M <= 8 else emu_lib.gemm_q8_1
        ref_m, env_m = oracle.gemv_q8_1(fmt, p, N, K, xq[:M * K // 32 * 36], M)
        y, rc, msg, guards = run(idx, p, N, K, xq[:M * K // 32 * 36], M)
        assert rc == 0 and guards, msg
        linear_check(y, ref_m, env_m, K, f"{fmt} M={M}")


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q8_0", "gguf:mxfp4", "nvfp4", "gguf:iq2_s", "gguf:tq1_0"])
@pytest.mark.parametrize("chunk,max_wgs", [(5, 1), (3, 2), (64, 3), (700, 3), (2900, 2), (700, 16), (2900, 8)])
def test_emulated_chunks(fmt, chunk, max_wgs):
    """Several launch chunks, each with several staged tiles and a partial
    one; small resident-workgroup counts make the launcher pick large tiles."""
    info = nq.format_query(fmt)
    B = info.block_values
    nblocks = 300 if chunk < 100 else 5000
    p = synth.payload(fmt, nblocks, 5, RECIPE)
    got, bad, msg, guards = emu_lib.decode(info.id, p, nblocks, B, "bf16", mis=3, chunk=chunk,
                                           max_wgs=max_wgs)
    assert bad == 0, msg
    assert guards
    assert _same(got, _oracle(fmt, p, nblocks, B, "bf16"), "bf16")


@pytest.mark.parametrize("upt", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("fmt", FORMATS)
def test_emulated_exact_tile_multiples(fmt, upt):
    """Payloads that end exactly at a tile boundary, at every payload
    alignment: the last full tile's 16-byte staging chunks may pass the
    payload's end, so that tile must be decoded without staging."""
    info = nq.format_query(fmt)
    B = info.block_values
    bpt = emu_lib.tile_blocks(info.id, upt)
    assert bpt > 0
    for nblocks, max_wgs in ((bpt, 1), (2 * bpt, 1), (3 * bpt, 2), (bpt + 1, 1), (2 * bpt - 1, 2)):
        p = synth.payload(fmt, nblocks, 11 + nblocks, RECIPE)
        ref = _oracle(fmt, p, nblocks, B, "bf16")
        for mis in range(4):
            got, bad, msg, guards = emu_lib.decode(info.id, p, nblocks, B, "bf16", mis=mis, max_wgs=max_wgs,
                                                   upt=upt)
            assert bad == 0, (nblocks, mis, msg)
            assert guards
            assert _same(got, ref, "bf16"), (nblocks, mis)


@pytest.mark.parametrize("upt", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("fmt", FORMATS)
def test_emulated_tile_sizes(fmt, upt):
    """Every tile size, over several tiles plus a partial one, to f32 and
    bf16."""
    info = nq.format_query(fmt)
    B = info.block_values
    nblocks = 5 * emu_lib.tile_blocks(info.id, upt) + 3
    p = synth.payload(fmt, nblocks, 21 + upt, RECIPE)
    for dtype in ("f32", "bf16"):
        got, bad, msg, guards = emu_lib.decode(info.id, p, nblocks, B, dtype, mis=1, max_wgs=2, upt=upt)
        assert bad == 0, msg
        assert guards
        assert _same(got, _oracle(fmt, p, nblocks, B, dtype), dtype)


# The launcher's tile size for long launches, per format (upt_long in nq_kernel.h).
UPT_CAP = {f: 2 for f in FORMATS}
UPT_CAP.update({f: 4 for f in ("gguf:q5_0", "gguf:q1_0", "gguf:q2_0", "nvfp4")})
UPT_CAP.update({f: 8 for f in ("gguf:q2_k", "gguf:q3_k", "gguf:iq2_xxs", "gguf:iq2_xs", "gguf:iq3_xxs", "gguf:iq1_s",
                               "gguf:iq3_s", "gguf:iq2_s", "gguf:iq1_m", "gguf:tq1_0", "gguf:tq2_0")})
BIG_CODEBOOK = ("gguf:iq2_s", "gguf:iq1_s", "gguf:iq1_m")
UPT_WIDE = BIG_CODEBOOK + ("gguf:iq2_xs", "gguf:iq3_s")  # 16-unit tiles from 3072 units per resident workgroup


def test_tile_size_by_rounds():
    """The launcher's tile size for [rows, 4096] tensors with 2048 resident
    workgroups (units = rows * 512; tiles = units / (256 * upt)): 1 below 128
    units per resident workgroup; the long-launch size L when its tiles fill
    the device four times over; otherwise the smallest of 2, 4, 8 whose tiles
    fit in one round (4, 8 for "nvfp4"), else L.  Large codebooks step up by
    units per resident workgroup alone, to at most 8; the widest-codebook
    formats and IQ3_S take 16 from 3072 units per resident workgroup."""
    g = 2048
    # rows -> choice, for L = 2, 4, 8
    by_rows = {
        256: (1, 1, 1),       # q = 64
        512: (2, 2, 2),       # q = 128: tiles(2) = 512 fit
        2048: (2, 2, 2),      # tiles(2) = 2048 = one round
        2049: (4, 4, 4),      # tiles(2) = 2049 > 2048, tiles(4) fit
        3072: (4, 4, 4),
        4096: (4, 4, 4),      # tiles(4) = 2048
        4097: (8, 8, 8),
        6144: (8, 8, 8),
        8192: (2, 8, 8),      # tiles(2) = 8192 = 4 rounds; L = 4: 4096 tiles, one fits at 8
        8193: (2, 4, 8),      # no size fits in one round: L
        14336: (2, 4, 8),
        16384: (2, 4, 8),     # L = 4: tiles(4) = 8192, four rounds
        1 << 20: (2, 4, 8),
    }
    big = {256: 1, 512: 2, 1023: 2, 1024: 4, 2047: 4, 2048: 8, 12287: 8, 12288: 16, 14336: 16, 1 << 20: 16}
    for fmt in FORMATS:
        fid = nq.format_query(fmt).id
        col = {2: 0, 4: 1, 8: 2}[UPT_CAP[fmt]]
        table = big if fmt in BIG_CODEBOOK else {r: w[col] for r, w in by_rows.items()}
        if fmt == "nvfp4":  # one-round choices start at 4
            table = {r: (4 if w == 2 else w) for r, w in table.items()}
        if fmt in UPT_WIDE:  # q = rows / 4 >= 3072
            table = {r: (16 if r >= 4 * 3072 else w) for r, w in table.items()}
        for rows, want in table.items():
            assert emu_lib.choose_upt(fid, rows * 512, g) == want, (fmt, rows)
        assert emu_lib.choose_upt(fid, 100, 0) == 1


@pytest.mark.parametrize("d_w", [1.0, 3.0, 448.0, 1e-30, 3e38, -3.0, -0.0, 0.0, float("inf"), float("-inf"),
                                 float("nan"), -1e-38])
def test_emulated_nvfp4_divisor(d_w):
    """Valid divisors and the words section 3.3 refuses (negative, zero,
    infinite, NaN, subnormal): the table's magnitudes with the divisor's sign
    inserted give the oracle's quotients (NaN by class)."""
    info = nq.format_query("nvfp4")
    p = synth.payload("nvfp4", 40, 3, RAW, divisor=d_w)
    for upt in (0, 2, 8):
        got, bad, msg, guards = emu_lib.decode(info.id, p, 40, 64, "f32", mis=2, upt=upt)
        assert bad == 0 and guards, msg
        assert _same(got, _oracle("nvfp4", p, 40, 64, "f32"), "f32"), (d_w, upt)


def test_nvfp4_table_from_two_quotients_per_scale():
    """The kernels build the 1024-entry quotient table from one division per
    scale magnitude and E2M1 class, scaled by powers of two; every entry must
    equal its own correctly rounded division, for every scale word and
    divisors of every binade and class: random words over the whole binary32
    range, the valid range [1, 448], subnormals, powers of two near the
    overflow and underflow edges, zeros, infinities and NaNs."""
    rng = np.random.default_rng(5)
    words = [rng.integers(0, 2 ** 32, size=40000, dtype=np.uint64).astype(np.uint32),
             rng.integers(0x3F800000, 0x43E00001, size=20000, dtype=np.uint64).astype(np.uint32),
             rng.integers(1, 0x00800000, size=5000, dtype=np.uint64).astype(np.uint32)]
    edges = []
    for e in list(range(0, 12)) + list(range(100, 150)) + list(range(240, 255)):
        for m in (0, 1, 0x400000, 0x7FFFFF):
            edges.append((e << 23) | m)
    edges += [0, 0x7F800000, 0x7FC00000, 0x7F800001, 0x00000001, 0x00800000, 0x3F800000, 0x43E00000]
    words.append(np.array(edges, dtype=np.uint32))
    words = np.concatenate(words)
    words = np.concatenate([words, words ^ np.uint32(0x80000000)])
    quad, direct = emu_lib.nvfp4_tables(words)
    qn = ((quad & 0x7F800000) == 0x7F800000) & ((quad & 0x007FFFFF) != 0)
    dn = ((direct & 0x7F800000) == 0x7F800000) & ((direct & 0x007FFFFF) != 0)
    bad = (qn != dn) | (~dn & (quad != direct))
    assert not bad.any(), f"{int(bad.sum())} entries differ, first divisor word {int(words[np.nonzero(bad.any(1))[0][0]]):#010x}"


@pytest.mark.parametrize("upt", [0, 2, 8])
def test_emulated_nvfp4_stacked_signed_divisors(upt):
    """Stacked divisors of both signs, zeros, an infinity and a NaN: tiles
    that start in a negative group read the table with the sign inserted,
    units past it divide directly."""
    d_ws = [3.0, -3.0, -0.0, 0.0, float("inf"), -448.0, float("nan"), 1.0]
    rows, K = 64, 128
    nb = rows * K // 64
    p = synth.payload("nvfp4", nb, 77, RAW, divisor=d_ws, divisors=len(d_ws))
    ref = oracle.decode_nvfp4_stacked(p, [rows, K], len(d_ws), "f32")
    fid = nq.format_query("nvfp4").id
    got, bad, msg, guards = emu_lib.decode(fid, p, nb, 64, "f32", mis=1, upt=upt, ndiv=len(d_ws))
    assert bad == 0 and guards, msg
    assert _same(got, ref, "f32")


@pytest.mark.parametrize("upt", [0, 1, 2, 8, 16])
@pytest.mark.parametrize("rows,K,divisors", [(24, 128, 1), (24, 128, 2), (24, 128, 3), (24, 128, 24),
                                             (40, 64, 40), (40, 64, 8), (6, 4096, 3), (96, 512, 4)])
def test_emulated_nvfp4_stacked_divisors(rows, K, divisors, upt):
    """Planes stacked from several sources: tiles that start in one divisor
    group and reach others (down to one-row groups of 8 units), at every
    payload alignment, against the oracle."""
    nb = rows * K // 64
    p = synth.payload("nvfp4", nb, 900 + divisors, RECIPE, divisors=divisors)
    ref = oracle.decode_nvfp4_stacked(p, [rows, K], divisors, "f32")
    fid = nq.format_query("nvfp4").id
    for mis in range(4):
        got, bad, msg, guards = emu_lib.decode(fid, p, nb, 64, "f32", mis=mis, upt=upt, ndiv=divisors)
        assert bad == 0, (mis, msg)
        assert guards
        assert _same(got, ref, "f32"), (mis, divisors)


@pytest.mark.parametrize("kind,fmt", [(0, "fp8_e4m3fn_row_bf16"), (1, "fp8_e4m3fn_row_fp16")])
@pytest.mark.parametrize("N,K,chunk", [(7, 48, 0), (5, 33, 0), (3, 1, 0), (1, 4099, 0), (9, 7, 0), (33, 256, 1000),
                                       (6, 100, 77), (1, 5000, 4096), (40, 16, 160), (70, 300, 0),
                                       (70, 300, 9000), (3, 40000, 0)])
def test_emulated_fp8_row(kind, fmt, N, K, chunk):
    """Row-scaled FP8: rows shorter and longer than a thread's 16 values,
    rows that start inside a thread, partial last threads, launches split
    mid-row, every payload alignment and output type."""
    rng = np.random.default_rng(N * 1000 + K)
    codes = rng.integers(0, 256, size=N * K, dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=N, dtype=np.uint16)
    p = np.concatenate([codes, scales.astype("<u2").view(np.uint8)])
    for dtype in ("f32", "bf16", "f16", "f64"):
        ref = oracle.decode_fp8_row(fmt, p, [N, K], dtype)
        for mis in range(4):
            # Outputs off 16-byte alignment by one element (the ABI refuses
            # outputs not aligned to their element size).
            got, bad, msg, guards = emu_lib.decode_fp8_row(kind, p, N, K, dtype, mis=mis,
                                                           out_mis=emu_lib.OSIZE[dtype] * (mis & 1), chunk=chunk)
            assert bad == 0, (mis, msg)
            assert guards
            assert _same(got, ref, dtype), (dtype, mis)


def test_fp8_row_division_by_multiplication():
    """The multiply-shift row division equals floor(n / d) for 31-bit n and
    every d up to 2^30: all d < 2^12, powers of two and their neighbours,
    random d; n at 0, 1, d - 1, d, d + 1, around multiples of d, near 2^31."""
    rng = np.random.default_rng(5)
    ds = set(range(1, 1 << 12)) | {1 << k for k in range(31)} | {(1 << k) + 1 for k in range(30)}
    ds |= {(1 << k) - 1 for k in range(2, 31)} | set(int(x) for x in rng.integers(1, 1 << 30, 3000))
    top = (1 << 31) - 1
    for d in sorted(ds):
        q = top // d
        ns = {0, 1, d - 1, d, d + 1, top, top - 1, q * d, q * d - 1, (q // 2) * d, (q // 2) * d - 1}
        ns |= set(int(x) for x in rng.integers(0, 1 << 31, 8))
        for n in ns:
            if 0 <= n <= top:
                assert emu_lib.f8_div(n, d) == n // d, (n, d)


def _gq_source(rng, N, K, in_dtype):
    x = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-30, 10, (N, 1)))).astype(np.float32)
    x[0, : min(K, 40)] = 0.0
    if in_dtype == "f32":
        return x, x
    if in_dtype == "f64":
        x64 = x.astype(np.float64) * (1 + 2.0 ** -30)
        return x64, x64
    import torch
    t = torch.from_numpy(x).to(torch.float16 if in_dtype == "f16" else torch.bfloat16)
    w = t.view(torch.int16).numpy().view(np.uint16)
    return w, w


@pytest.mark.parametrize("scheme", ["q4_g64_fp16", "q5_g64_fp16", "q6_g64_fp16", "q8_g32_fp16"])
@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16", "f64"])
def test_emulated_grouped_absmax(scheme, in_dtype):
    """The encoder's lane code against the oracle: full and short last groups,
    rows not a multiple of 8 or 4 values, rows shorter than a lane's 8 values,
    aligned and misaligned sources and code outputs (vector and element
    paths), zero groups, tiny (rescued) and large scales."""
    sid, G, _, _ = oracle.GQ_SCHEMES[scheme]
    code = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}[in_dtype]
    esz = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8}[in_dtype]
    rng = np.random.default_rng(sid * 10 + code)
    for N, K in ((5, 4 * G), (3, 3 * G + 24), (4, 70), (6, 13), (2, 5), (1, G), (9, 2 * G + 3)):
        x, ox = _gq_source(rng, N, K, in_dtype)
        want = oracle.grouped_absmax(scheme, ox, in_dtype)
        for x_mis, c_mis in ((0, 0), (esz, 1), (0, 2)):
            st, codes, scales, bad, msg, guards = emu_lib.grouped_absmax(sid, G, x, code, x_mis, c_mis)
            assert bad == 0, (N, K, x_mis, msg)
            assert guards
            assert st == want[0] == 0
            assert np.array_equal(codes, want[1]), (N, K, x_mis, c_mis)
            assert np.array_equal(scales, want[2]), (N, K, x_mis, c_mis)


def test_emulated_grouped_absmax_failures():
    """Non-finite sources and scales past binary16 set the same status bits as
    the oracle (other groups still encode)."""
    x = np.ones((3, 64), np.float32)
    x[1, 5] = np.inf
    x[2, 9] = 8321040.0  # raw scale 65520 for q8 -> binary16 infinity
    for scheme in ("q8_g32_fp16", "q4_g64_fp16"):
        sid, G, _, _ = oracle.GQ_SCHEMES[scheme]
        st, codes, scales, bad, msg, guards = emu_lib.grouped_absmax(sid, G, x, 0)
        want = oracle.grouped_absmax(scheme, x)
        assert bad == 0 and guards
        assert st == want[0]
        assert np.array_equal(codes[0], want[1][0]) and np.array_equal(scales[0], want[2][0])
    assert emu_lib.grouped_absmax(3, 32, x, 0)[0] == 3


# --------------------------------------------------------------------------
# Products with q8_1 activations and the q8_1 quantizer, through the
# kernels' lane code on the CPU: every weight read is bounds-checked, the
# output guards must hold, the product meets the oracle's criterion and the
# quantizer matches the oracle bit for bit.
# --------------------------------------------------------------------------
from linear_criterion import check as linear_check  # noqa: E402

GGUF = [f for f in FORMATS if f.startswith("gguf:")]


def _act(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * 2.0
    x[:, rng.integers(0, K, size=max(1, K // 61))] *= 30.0
    return x


@pytest.mark.parametrize("fmt", GGUF)
def test_emu_gemv_matches_oracle(fmt):
    idx, B, S, _ = oracle.info(fmt)
    K = 2 * max(B, 256)
    for N, M, w_mis, resident, max_rows in [(13, 1, 0, 2048, 0), (11, 2, 3, 1, 0), (9, 3, 1, 2048, 4),
                                            (6, 8, 2, 2, 5)]:
        w = synth.payload(fmt, N * K // B, 91 + N, synth.binade(-6, -2, False))
        _, xq = oracle.quantize_q8_1(_act(M, K, N).astype(np.float32))
        y, rc, msg, guards = emu_lib.gemv_q8_1(idx, w, N, K, xq, M, w_mis=w_mis, resident=resident,
                                               max_rows=max_rows)
        assert rc == 0, msg
        assert guards
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} N={N} M={M}")


@pytest.mark.parametrize("fmt", GGUF)
def test_emu_gemv_single_round_matches_oracle(fmt):
    """The single-round kernel on a device of one compute unit holding
    per_cu workgroups of up to 16 waves: phase 1 moves the activation blocks
    (the last act_dw mod 4 dwords by dword loads) and the codebook tables
    into LDS, spread over the workgroup's waves; each wave's chunk of 1, 2 or
    3 whole rows is staged by aligned 16-byte loads to LDS (the launch's last
    group shifted into place when the payload ends inside it).  Whole rows
    per chunk grow when more waves than one workgroup of 16 (or per_cu of
    them) would be needed.  Several activation rows are read from global
    memory by four-wave workgroups (two rows per chunk first once there are
    16 or more rows); misaligned weight bytes and launches that do not fit
    take the chunk loop."""
    idx, B, S, _ = oracle.info(fmt)
    K = 3 * B if B >= 64 else 7 * B
    for N, M, per_cu, w_mis, rw in [(12, 1, 1, 0, 1), (20, 1, 1, 0, 2), (40, 1, 1, 0, 3), (60, 1, 1, 0, 0),
                                    (39, 1, 2, 0, 2), (12, 1, 3, 4, 0), (13, 3, 2, 0, 2), (12, 8, 1, 0, 3),
                                    (5, 2, 1, 0, 2), (17, 4, 8, 0, 2), (33, 4, 1, 0, 0), (7, 4, 4, 0, 1)]:
        w = synth.payload(fmt, N * K // B, 17 + N + M, synth.binade(-6, -2, False))
        _, xq = oracle.quantize_q8_1(_act(M, K, N + 3).astype(np.float32))
        y, rc, msg, guards, got = emu_lib.gemv_q8_1(idx, w, N, K, xq, M, w_mis=w_mis, gv1_cus=1,
                                                    gv1_per_cu=per_cu, with_rw=True)
        assert rc == 0, msg
        assert guards
        assert got == rw, (N, M, per_cu, w_mis)
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} N={N} M={M} rows per chunk {rw}")


def _items_per_block(fmt):
    """Items of the product's integer path per block: 64-value items for
    q4_k, q5_k and q6_k, 32-value items otherwise."""
    B = oracle.info(fmt)[1]
    return B // 64 if fmt in ("gguf:q4_k", "gguf:q5_k", "gguf:q6_k") else B // 32


@pytest.mark.parametrize("fmt", GGUF)
def test_emu_gemv_row_split_matches_oracle(fmt):
    """Single-round launches whose rows hold more than 64 items: each row is
    split in two parts (blocks 0 .. cb - 1 and cb .. nbr - 1, cb =
    ceil(nbr / 2)) taken by two waves of one workgroup, and part 0's wave
    adds the two row sums.  Odd block counts give unequal parts; the longer
    rows give each lane several items per part; 9 rows (18 parts) take two
    workgroups of 10 waves, the second with one empty row.  (Several
    activation rows keep whole rows.)"""
    idx, B, S, _ = oracle.info(fmt)
    ipb = _items_per_block(fmt)
    for nbr, N, M in [(64 // ipb + 1, 5, 1), (64 // ipb + 1, 9, 1), (2 * (64 // ipb) + 3, 3, 1),
                      (2 * (64 // ipb) + 3, 6, 1)]:
        K = nbr * B
        w = synth.payload(fmt, N * nbr, 23 + N + nbr, synth.binade(-6, -2, False))
        _, xq = oracle.quantize_q8_1(_act(M, K, N + nbr).astype(np.float32))
        y, rc, msg, guards, rw, ks = emu_lib.gemv_q8_1(idx, w, N, K, xq, M, gv1_cus=1, gv1_per_cu=8, with_rw=True,
                                                       with_parts=True)
        assert rc == 0, msg
        assert guards
        assert (rw, ks) == (1, 2), (nbr, N, M)
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} N={N} K={K} M={M} split rows")


@pytest.mark.parametrize("fmt,N,K,M,rw,ks", [("gguf:q4_k", 14336, 4096, 1, 2, 1), ("gguf:q4_k", 4096, 14336, 1, 1, 2),
                                             ("gguf:q4_k", 4096, 4096, 8, 2, 1), ("gguf:q6_k", 1024, 4096, 8, 1, 1),
                                             ("gguf:q8_0", 14336, 4096, 1, 0, 0),
                                             ("gguf:q6_k", 4096, 14336, 1, 0, 0), ("gguf:q4_0", 1024, 4096, 1, 1, 2),
                                             ("gguf:iq2_xxs", 14336, 4096, 1, 2, 1),
                                             ("gguf:iq4_xs", 4096, 14336, 1, 1, 2),
                                             ("gguf:q4_k", 1024, 4096, 1, 1, 1),
                                             ("gguf:q4_0", 4096, 4096, 1, 1, 1),
                                             ("gguf:mxfp4", 2048, 4096, 1, 1, 2)])
def test_emu_gemv_single_round_plan(fmt, N, K, M, rw, ks):
    """On a device of 256 compute units holding up to 8 workgroups, 160 KiB
    of LDS and 32 waves each, the single-round plan takes the fewest rows per
    chunk whose chunks all fit at once, or, for several activation rows and
    at least 4096 rows, two rows first; single-row chunks of rows with more
    than 64 items split each row in two parts first when K >= 8192 or whole
    rows would give fewer than 16 waves per unit (q4_k and iq4_xs with 14336
    columns, q4_0 and mxfp4 with 1024 or 2048 rows of 4096), not at [4096,
    4096]; a q4_k row of 4096 columns (64 items) stays whole.  With one activation row, workgroups hold up to 16 waves
    (the activation copy in LDS serves them all), as many workgroups per
    unit as fit; several activation rows take four-wave workgroups.  Weights
    too large for one round (q8_0 at [14336, 4096]: 62 MB) take the chunk
    loop."""
    idx, B, S, _ = oracle.info(fmt)
    p = emu_lib.gemv1_plan(idx, N, K, M)
    assert (p[0], p[4]) == (rw, ks), p
    if rw:
        nbr = K // B
        cb = -(-nbr // ks)
        assert p[5] == cb
        chunk_bytes = rw * nbr * S if ks == 1 else cb * S
        assert p[1] == 4 * ((15 + chunk_bytes + 15) // 16 + 1)
        nw, act_dw = p[6], p[7]
        assert act_dw == ((K // 32) * 9 if M == 1 else 0)
        act_region = -(-act_dw // 4) * 4
        assert p[2] == 4 * (act_region + nw * p[1])
        chunks = -(-N // rw) if ks == 1 else N * ks
        assert 1 <= nw <= 16 and nw % ks == 0
        assert p[3] == -(-chunks // nw)
        g = -(-p[3] // 256)  # workgroups per compute unit
        assert g <= min(8, 163840 // p[2], 32 // nw)
        # the fewest workgroups per compute unit: with one fewer, a workgroup
        # would need more than 16 waves or would not fit
        if M > 1:
            assert nw == 4
        else:
            # the most workgroups per compute unit (the smallest workgroups):
            # with one more per unit, they would not all fit at once
            g = max(gg for gg in range(1, 9) if -(-chunks // (256 * gg)) + (-(-chunks // (256 * gg))) % ks == nw)
            assert nw == -(-chunks // (256 * g)) + (-(-chunks // (256 * g))) % ks
            for g1 in range(g + 1, 9):
                nw1 = -(-chunks // (256 * g1))
                nw1 += nw1 % ks
                lds1 = 4 * (act_region + nw1 * p[1])
                assert nw1 > 16 or lds1 > 163840 or min(8, 163840 // lds1, 32 // nw1) < g1
    assert emu_lib.gemv1_plan(idx, N, K, M, w_mis=8)[0] == 0


def _kquant_scale_min(q, j):
    """Sub-block j's 6-bit scale and min from the 12 packed bytes of a q4_k /
    q5_k block (DequantizePacked, "Mathematical decoding rules", Q4_K): for j
    < 4 the low 6 bits of bytes j and j + 4; otherwise the low nibble (scale)
    or high nibble (min) of byte j + 4 with the top two bits of byte j - 4
    (scale) or j (min) above it."""
    if j < 4:
        return q[j] & 63, q[j + 4] & 63
    return (q[j + 4] & 15) | ((q[j - 4] >> 6) << 4), (q[j + 4] >> 4) | ((q[j] >> 6) << 4)


def test_emu_kq_scale_min_pair():
    """The product's byte-select rule for the scale and min pair of a 64-value
    item equals the per-sub-block rule, on random scale fields and on fields
    with every bit set or clear (both halves of each byte, both item pairs
    per half)."""
    rng = np.random.default_rng(0x5C41E)
    fields = [rng.integers(0, 256, 12, dtype=np.uint8) for _ in range(3000)]
    fields += [np.full(12, v, np.uint8) for v in (0x00, 0xFF, 0xC0, 0x3F, 0x0F, 0xF0, 0x55, 0xAA)]
    for q in fields:
        q = [int(v) for v in q]
        for g in range(4):
            s0, m0 = _kquant_scale_min(q, 2 * g)
            s1, m1 = _kquant_scale_min(q, 2 * g + 1)
            assert emu_lib.kq_scale_min_pair(bytes(q), g) == (s0, s1, m0, m1), (q, g)


def test_emu_gemv_rejects_nvfp4_with_divisor():
    y, rc, _, _ = emu_lib.gemv_q8_1(nq.format_query("nvfp4").id, np.zeros(40, np.uint8), 1, 64,
                                    np.zeros(72, np.uint8), 1)
    assert rc == -1


@pytest.mark.parametrize("in_dtype,code", [("f32", 0), ("f16", 1), ("bf16", 2), ("f64", 3)])
def test_emu_quantize_q8_1_matches_oracle(in_dtype, code):
    M, K = 3, 352
    x = _act(M, K, 5)
    x[1, 64:96] = 0.0                 # an all-zero block
    x[2, 160] = 1e-30                 # a tiny block
    x[0, 96:128] = 65024.0            # a block whose sum overflows binary16
    if in_dtype == "f32":
        xs = x.astype(np.float32)
    elif in_dtype == "f16":
        xs = x.astype(np.float16).view(np.uint16)
    elif in_dtype == "bf16":
        xs = oracle.convert(x.astype(np.float32), "bf16").reshape(M, K)
    else:
        xs = x
    ost, ob = oracle.quantize_q8_1(xs, in_dtype)
    assert ost == 4
    esz = xs.dtype.itemsize
    for mis in sorted({0, esz, 2 * esz, 8}):
        st, b, rc, msg, guards = emu_lib.quantize_q8_1(xs, code, x_mis=mis, chunk=5)
        assert rc == 0, msg
        assert guards
        assert st == ost
        assert np.array_equal(b, ob), f"{in_dtype} mis={mis}"


def test_emu_quantize_q8_1_failures():
    x = _act(2, 96, 3).astype(np.float32)
    x[0, 3] = np.nan
    x[1, 70] = 2.0 ** 23
    ost, ob = oracle.quantize_q8_1(x)
    st, b, rc, msg, guards = emu_lib.quantize_q8_1(x, 0)
    assert rc == 0 and guards
    assert st == ost == 3
    assert np.array_equal(b, ob)


@pytest.mark.parametrize("fmt,K", [("gguf:q8_0", 16384), ("gguf:q4_k", 28672), ("gguf:q6_k", 16384),
                                   ("gguf:q4_1", 24576), ("gguf:iq4_xs", 24576)])
def test_emu_gemv_rows_staged_in_chunks(fmt, K):
    """Rows longer than one staged chunk are staged and summed chunk by chunk."""
    idx, B, S, _ = oracle.info(fmt)
    assert K // B * S > 12288
    N, M = 3, 2
    w = synth.payload(fmt, N * K // B, 5, synth.binade(-6, -2, False))
    _, xq = oracle.quantize_q8_1(_act(M, K, 8).astype(np.float32))
    y, rc, msg, guards = emu_lib.gemv_q8_1(idx, w, N, K, xq, M, w_mis=1)
    assert rc == 0, msg
    assert guards
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    linear_check(y, ref, env, K, fmt)


@pytest.mark.parametrize("fmt,K", [("gguf:q8_0", 160), ("gguf:q4_0", 96), ("gguf:q4_1", 224), ("gguf:iq4_nl", 32),
                                   ("gguf:mxfp4", 288), ("gguf:nvfp4", 192)])
def test_emu_gemv_k_not_a_multiple_of_128(fmt, K):
    """The activation's LDS layout is swizzled only when K is a multiple of
    128; other K take the plain layout."""
    idx, B, S, _ = oracle.info(fmt)
    N, M = 7, 3
    w = synth.payload(fmt, N * K // B, 21, synth.binade(-6, -2, False))
    _, xq = oracle.quantize_q8_1(_act(M, K, 4).astype(np.float32))
    y, rc, msg, guards = emu_lib.gemv_q8_1(idx, w, N, K, xq, M, w_mis=3)
    assert rc == 0, msg
    assert guards
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    linear_check(y, ref, env, K, fmt)


# --------------------------------------------------------------------------
# Batched products on the matrix cores (more than 8 activation rows): the
# workgroups' staging, the lanes' operands and scaling around an emulated
# 16 x 16 x 32 8-bit matrix instruction, bounds-checked weight reads, every
# tile met exactly once.
# --------------------------------------------------------------------------
GEMM_FMTS = GGUF


def _gemm_k(B):
    """K that leaves a partial last K step (256 values) where the block size allows."""
    return 352 if B == 32 else 384 if B in (64, 128) else 768


def _sp4_planned(N, M, cus, nsplit):
    """4-span K steps: 64-row tiles, more than two per compute unit, or five
    eighths to two per compute unit with K split."""
    bm = 16 if M <= 16 else 32 if M <= 32 else 64
    tiles = -(-N // 128) * -(-M // bm)
    return cus > 0 and bm == 64 and (tiles > 2 * cus or (5 * cus <= 8 * tiles < 16 * cus and nsplit >= 2))


@pytest.mark.parametrize("fmt", GEMM_FMTS)
def test_emu_gemm_matches_oracle(fmt):
    """Every gguf format over ragged tiles and K steps, launch limits, both
    K step lengths (cus = 1 plans 4-span steps for grids of more than two
    64-row tiles), with and without the per-call rewrite."""
    idx, B, S, _ = oracle.info(fmt)
    K = _gemm_k(B)
    for N, M, w_mis, max_rows, max_mrows, cus in [(150, 9, 0, 0, 0, 0), (37, 70, 1, 0, 0, 0),
                                                  (260, 65, 3, 128, 0, 256), (130, 100, 2, 0, 40, 1),
                                                  (37, 1100, 1, 0, 500, 256), (140, 1030, 2, 128, 0, 1),
                                                  (60, 32, 1, 0, 0, 0), (200, 21, 3, 0, 0, 256),
                                                  (140, 16, 2, 0, 0, 0), (37, 7, 1, 0, 0, 256),
                                                  (300, 130, 1, 0, 0, 1)]:
        w = synth.payload(fmt, N * K // B, 7 + N, synth.binade(-6, -2, False))
        _, xq = oracle.quantize_q8_1(_act(M, K, M).astype(np.float32))
        y, rc, msg, guards, (ns, once, sp4) = emu_lib.gemm_q8_1(idx, w, N, K, xq, M, w_mis=w_mis,
                                                                 max_rows=max_rows, max_mrows=max_mrows, cus=cus,
                                                                 with_splits=True)
        assert rc == 0, msg
        assert guards
        assert once == (cus > 0 and M > 256)
        assert sp4 == _sp4_planned(N, M, cus, ns)
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} N={N} M={M} rewritten once={once} 4-span steps={sp4}")


def test_emu_gemm_tile_order_covers_every_tile():
    """Grids that are not multiples of the 8 XCDs: every tile once (checked by
    the emulator) and the product right."""
    fmt = "gguf:q8_0"
    idx, B, S, _ = oracle.info(fmt)
    K = 64
    for N, M in [(1100, 200), (1025, 9), (129, 577)]:
        w = synth.payload(fmt, N * K // B, N, synth.binade(-6, -2, True))
        _, xq = oracle.quantize_q8_1(_act(M, K, 3).astype(np.float32))
        y, rc, msg, guards = emu_lib.gemm_q8_1(idx, w, N, K, xq, M)
        assert rc == 0, msg
        assert guards
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} N={N} M={M}")



@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q8_0", "gguf:q6_k", "gguf:q2_k", "gguf:iq2_xs", "gguf:q4_1"])
def test_emu_gemm_split_k(fmt):
    """K split over workgroups (planned for a small device), partials summed in
    split order: the criterion holds; every tile and split is met once.  The
    last shape has five eighths to two 64-row tiles per compute unit (9 on
    8): three splits in 4-span K steps; the second (4 on 16) stays in 8-span
    steps."""
    idx, B, S, _ = oracle.info(fmt)
    for N, K, M, cus in [(200, 4096, 20, 64), (130, 2304, 70, 16), (300, 2304, 130, 8)]:
        w = synth.payload(fmt, N * K // B, N + M, synth.binade(-6, -2, False))
        _, xq = oracle.quantize_q8_1(_act(M, K, 6).astype(np.float32))
        y, rc, msg, guards, (ns, once, sp4) = emu_lib.gemm_q8_1(idx, w, N, K, xq, M, w_mis=1, cus=cus,
                                                                 with_splits=True)
        assert rc == 0, msg
        assert guards
        assert ns >= 2
        assert not once and sp4 == (cus == 8)
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} N={N} K={K} M={M} splits={ns}")


def _up(x):
    return -(-x // 256) * 256


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "gguf:q6_k", "gguf:q8_0"])
def test_emu_gemm_plan_invariants(fmt):
    """The batched product's plan on 256 compute units at Llama-3-8B shapes:
    the tile height follows M; the K splits cover K with none empty (at least
    4 steps each, partials at most 2 GiB, only below two tiles per compute
    unit; 64-row tiles in 8-span steps within 512 workgroups); 4-span steps
    only with 64-row tiles; the weight rewritten once
    exactly above 384 rows for q4_k and 256 for the others; the workspace is the partials plus the rewritten
    codes, scales and (q4_k) offsets, each rounded up to 256 bytes; without
    a workspace the plan is unsplit, in 8-span steps where 4-span ones came
    with a split."""
    idx = oracle.info(fmt)[0]
    nh, aff = (2, False) if fmt == "gguf:q6_k" else (1, fmt == "gguf:q4_k")
    for N, K in [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (128256, 4096), (300, 1024)]:
        for M in [5, 16, 17, 32, 33, 64, 65, 128, 192, 256, 257, 384, 512, 768, 1024, 2048, 4096]:
            p = emu_lib.gemm_plan(idx, N, K, M, 256)
            bm = 16 if M <= 16 else 32 if M <= 32 else 64
            assert p["bm"] == bm
            tiles = -(-N // 128) * -(-M // bm)
            steps = -(-(K // 32) // p["sp"])
            assert p["sp"] in (4, 8) and (p["sp"] == 4) <= (bm == 64)
            assert p["nsplit"] * p["sps"] >= steps and (p["nsplit"] - 1) * p["sps"] < steps
            if p["nsplit"] > 1:
                assert tiles < 512 and p["sps"] >= 4 and p["nsplit"] * M * N * 4 <= 1 << 31
                if bm == 64 and p["sp"] == 8:
                    assert tiles * p["nsplit"] <= 512  # one pass of two workgroups per compute unit
            else:
                assert p["sps"] == steps
                assert (p["sp"] == 4) == (bm == 64 and tiles > 512)
            assert p["once"] == (M > (384 if fmt == "gguf:q4_k" else 256))
            ws = _up(p["nsplit"] * M * N * 4) if p["nsplit"] > 1 else 0
            if p["once"]:
                ws += _up(N * K) + _up(K // 32 * nh * N * 4) * (2 if aff else 1)
            assert p["ws"] == ws, (N, K, M)
            assert p["plain_nsplit"] == 1 and p["plain_sp"] == (p["sp"] if p["nsplit"] == 1 else 8)
            assert p["plain_sps"] == -(-(K // 32) // p["plain_sp"])
    # plans the measurements quote
    plan = lambda N, K, M: (lambda p: (p["nsplit"], p["sp"], p["bm"]))(emu_lib.gemm_plan(idx, N, K, M, 256))
    assert plan(14336, 4096, 512) == (1, 4, 64)     # 896 tiles
    assert plan(4096, 14336, 512) == (3, 4, 64)     # 256 tiles: three splits in 4-span steps
    assert plan(4096, 14336, 384) == (4, 4, 64)     # 192 tiles
    assert plan(4096, 14336, 320) == (3, 8, 64)     # 160 tiles: 8-span steps fill 480 of 512 slots
    assert plan(4096, 14336, 64) == (14, 8, 64)     # 32 tiles, 56 steps
    assert plan(14336, 4096, 16) == (4, 8, 16)      # 112 tiles of 16 rows
    assert plan(1024, 4096, 1100) == (3, 8, 64)     # 144 tiles: 3 splits (432 workgroups), not 4 (576)


@pytest.mark.parametrize("M", [3, 70])
def test_emu_products_over_non_finite_scales(M):
    """Rows with an infinite or NaN weight scale give non-finite outputs on
    both sides (which non-finite value may differ); the other rows meet the
    criterion (single-row kernel for 3 activation rows, matrix cores for 70)."""
    fmt, N, K = "gguf:q8_0", 40, 256
    idx, B, S, _ = oracle.info(fmt)
    w = synth.payload(fmt, N * K // B, 71, synth.binade(-6, -2, True)).copy()
    blk = w.reshape(N, K // 32, 34)
    blk[3, 1, 0:2] = [0x00, 0x7C]
    blk[5, 0, 0:2] = [0x00, 0x7E]
    _, xq = oracle.quantize_q8_1(_act(M, K, 72).astype(np.float32))
    ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
    run = emu_lib.gemv_q8_1 if M <= 8 else emu_lib.gemm_q8_1
    y, rc, msg, guards = run(idx, w, N, K, xq, M)
    assert rc == 0, msg
    assert guards
    bad = np.zeros(N, bool)
    bad[[3, 5]] = True
    assert not np.any(np.isfinite(y[:, bad])) and not np.any(np.isfinite(ref[:, bad]))
    linear_check(y[:, ~bad], ref[:, ~bad], env[:, ~bad], K, f"{fmt} finite rows")


@pytest.mark.parametrize("fmt,N,K,M", [("gguf:q8_0", 1, 32, 5), ("gguf:q8_0", 1, 32, 33), ("gguf:q4_k", 1, 256, 32),
                                       ("gguf:q2_k", 3, 256, 65), ("gguf:iq1_m", 2, 256, 6)])
def test_emu_gemm_tiny_shapes(fmt, N, K, M):
    """One weight row, one span or one block of K, activation rows at the
    tile-height boundaries."""
    idx, B, S, _ = oracle.info(fmt)
    w = synth.payload(fmt, N * K // B, N + K + M, synth.binade(-6, -2, False))
    _, xq = oracle.quantize_q8_1(_act(M, K, 11).astype(np.float32))
    for cus in (0, 256):
        y, rc, msg, guards = emu_lib.gemm_q8_1(idx, w, N, K, xq, M, w_mis=1, cus=cus)
        assert rc == 0, msg
        assert guards
        ref, env = oracle.gemv_q8_1(fmt, w, N, K, xq, M)
        linear_check(y, ref, env, K, f"{fmt} [{N}, {K}] x {M}")


# ---------------------------------------------------------------------------
# Many-tensor launches (nq_dequantize_packed_many): the launcher's packing
# into launches of at most 64 entries and the kernel's tile search, per tile.
# ---------------------------------------------------------------------------
def _many_case(fmt, counts, seed, dtype="bf16", vec=True, resident=2048, chunk=0):
    info = nq.format_query(fmt)
    B = info.block_values
    recipe = RECIPE if fmt == "nvfp4" else RAW
    payloads = [synth.payload(fmt, nb, seed + k, recipe) for k, nb in enumerate(counts)]
    vals, bad, msg, guards, launches, upts = emu_lib.decode_many(info.id, payloads, B, dtype, vec=vec,
                                                                 resident=resident, chunk=chunk)
    assert bad == 0, msg
    assert guards
    for k, (p, nb) in enumerate(zip(payloads, counts)):
        assert _same(vals[k], _oracle(fmt, p, nb, B, dtype), dtype), (fmt, k, nb)
    return launches, upts


@pytest.mark.parametrize("fmt", FORMATS)
def test_emulated_many_every_format(fmt):
    """Ragged tensors of one format, one launch; tiny device (resident 16)
    so the larger tensors take several 2-unit tiles."""
    launches, upts = _many_case(fmt, [1, 3, 37, 2, 64, 5], 90, resident=16)
    assert launches == 1 and upts == {2}


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "nvfp4", "gguf:q8_0", "gguf:iq2_s", "gguf:tq2_0"])
def test_emulated_many_launch_limits_and_tile_sizes(fmt):
    """130 tensors: three launches (64, 64, 2 entries); on a one-workgroup
    device the two full launches take the format's largest tiles and the last
    (2 small tensors) 2-unit tiles; on a large device every launch takes
    2-unit tiles."""
    counts = [1 + (7 * k) % 13 for k in range(128)] + [1, 1]
    launches, upts = _many_case(fmt, counts, 500, resident=1)
    assert launches == 3 and upts == {2, min(8, UPT_CAP[fmt])}
    launches, upts = _many_case(fmt, counts, 500, resident=1 << 20)
    assert launches == 3 and upts == {2}


@pytest.mark.parametrize("fmt", ["gguf:q4_0", "gguf:q6_k", "nvfp4", "gguf:tq1_0"])
@pytest.mark.parametrize("chunk", [1, 3, 40])
def test_emulated_many_tensors_split_into_chunks(fmt, chunk):
    """A tensor larger than a launch chunk takes several entries (each with the
    tensor's divisor for nvfp4); entries of one tensor can fall in two launches."""
    counts = [100, 7, 1, 129] + [2] * 60 + [77]
    launches, upts = _many_case(fmt, counts, 700, resident=1, chunk=chunk)
    entries = sum((c + chunk - 1) // chunk for c in counts)
    assert launches == (entries + 63) // 64


@pytest.mark.parametrize("dtype", ["f32", "f16", "f64"])
@pytest.mark.parametrize("fmt", ["gguf:q5_1", "gguf:iq3_xxs", "gguf:mxfp4", "nvfp4"])
def test_emulated_many_output_types_and_alignment(fmt, dtype):
    for vec in (True, False):
        launches, upts = _many_case(fmt, [4, 1, 33], 40, dtype=dtype, vec=vec, resident=1 << 20)
        assert upts == ({2} if vec and dtype != "f64" else {8})
