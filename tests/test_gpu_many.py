"""GPU (gfx950): several tensors decoded by one nq_dequantize_packed_many call.

Every output must equal the oracle's decode of its tensor bit for bit (NaN by
class), exactly as single-tensor calls do; tensors of one format share
launches of up to 64 entries, so the mixes below cross that limit, mix empty,
one-block, ragged and multi-tile tensors, 16-byte aligned and element-aligned
outputs, and keep a guard gap around every output to catch a write into a
neighbour's range.  The measurement kernel (nq_measure_stream) is checked
against the pattern its header specifies.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_nq_amd as nq
import compare
import oracle
import synth
from synth import workloads
from gpu_util import TORCH_DT, announce, oracle_blocks, to_numpy, upload

pytestmark = pytest.mark.gpu

FORMATS = oracle.format_names()
RAW = synth.raw()
RECIPE = synth.binade(-12, -6, True)
GUARD = 48  # elements of sentinel between outputs


def _sentinel(dtype):
    return float("nan")


class Mix:
    """Tensors with outputs carved from one buffer, separated by NaN guards."""

    def __init__(self, specs, dtype):
        self.dtype = dtype
        self.items = []
        total = GUARD
        layout = []
        for fmt, shape, seed, recipe, off in specs:
            nel = int(np.prod(shape)) if len(shape) else 1
            layout.append((total + off, nel))
            total += off + nel + GUARD
            total += (-total) % 8  # next output starts 16-byte aligned before its offset (bf16/f16: 8 elements)
        self.buf = torch.full((total,), _sentinel(dtype), dtype=TORCH_DT[dtype], device="cuda:0")
        for (fmt, shape, seed, recipe, off), (o, nel) in zip(specs, layout):
            info = nq.format_query(fmt)
            nb = nel // info.block_values
            p = synth.payload(fmt, nb, seed, recipe)
            payload, keep = upload(p, pay_off=seed % 4)
            self.items.append(dict(fmt=fmt, fid=info.id, shape=shape, p=p, payload=payload, keep=keep, o=o,
                                   nel=nel, out=self.buf[o:o + nel]))

    def descs(self):
        return [(it["fid"], it["payload"].data_ptr(), it["payload"].numel(), it["shape"], it["out"].data_ptr())
                for it in self.items]

    def run(self, stream=None):
        h = (stream or torch.cuda.current_stream()).cuda_stream
        st, failed = nq.dequantize_packed_many_raw(self.descs(), nq.DTYPE_CODES[self.dtype], h)
        torch.cuda.synchronize()
        return st, failed

    def check(self, what):
        host = to_numpy(self.buf, self.dtype)
        inside = np.zeros(host.size, dtype=bool)
        for k, it in enumerate(self.items):
            got = host[it["o"]:it["o"] + it["nel"]]
            ref = oracle.decode(it["fmt"], it["p"], it["shape"], self.dtype).ravel()
            assert compare.same(got, ref, self.dtype), \
                f"{what}: tensor {k} {it['fmt']} {it['shape']}: {compare.describe(got, ref, self.dtype)}"
            inside[it["o"]:it["o"] + it["nel"]] = True
        assert np.all(compare.nan_mask(host[~inside], self.dtype)), f"{what}: a write outside every output"


def _shape_for(rng, B, kind):
    if kind == 0:
        return [0, B]                                   # empty
    if kind == 1:
        return [B]                                      # one block
    if kind == 2:
        return [int(rng.integers(1, 5)), int(rng.integers(1, 40)) * B]   # ragged, rank 2
    if kind == 3:
        return [2, 3, int(rng.integers(1, 9)) * B]      # rank 3
    return [int(rng.integers(1, 4)) * 16384 // B + 1, B]   # one to three 16384-value tiles plus a block


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "f64"])
def test_many_every_format_mixed(dtype):
    """Every format three times (so each format's group has several entries),
    shapes from empty to multi-tile, outputs 16-byte aligned or shifted by one
    element, payloads at offsets 0..3, in one call."""
    rng = np.random.default_rng(1000 + len(dtype))
    specs = []
    for rep in range(3):
        for i, fmt in enumerate(FORMATS):
            B = nq.format_query(fmt).block_values
            kind = int(rng.integers(0, 5))
            recipe = RECIPE if fmt == "nvfp4" else (RAW if rep == 0 else RECIPE)
            off = 1 if (rep + i) % 4 == 3 else 0
            specs.append((fmt, _shape_for(rng, B, kind), 7000 + 97 * rep + i, recipe, off))
    mix = Mix(specs, dtype)
    announce(f"many: every format x3 -> {dtype}, {len(specs)} tensors")
    assert mix.run() == (0, -1)
    mix.check(f"every format -> {dtype}")


@pytest.mark.parametrize("fmt", ["gguf:q4_k", "nvfp4", "gguf:iq2_s", "gguf:tq1_0"])
def test_many_more_than_one_launch(fmt):
    """150 tensors of one format (three launches of at most 64 entries), each
    nvfp4 tensor with its own divisor; the second launch holds a [4096, 4096]
    tensor, enough units for the 8-units-per-thread tiles, the other two take
    the 2-unit tiles."""
    B = nq.format_query(fmt).block_values
    rng = np.random.default_rng(77)
    specs = [(fmt, [int(rng.integers(1, 40)), B], 300 + k, workloads.recipe_for(fmt), 0) for k in range(149)]
    specs.insert(70, (fmt, [4096, 4096], 299, workloads.recipe_for(fmt), 0))
    mix = Mix(specs, "bf16")
    announce(f"many: {fmt} x150 with one [4096, 4096]")
    assert mix.run() == (0, -1)
    mix.check(f"{fmt} x150")


def test_many_matches_single_calls_llama3_8b_layer():
    """One Llama-3-8B layer's seven tensors in each of the five formats of the
    weight-set workload (35 tensors, one call) give the bits of 35
    single-tensor calls."""
    specs = []
    for f in workloads.CONFIG5_ROTATION:
        for k, (name, shape) in enumerate(workloads.LLAMA3_8B_LAYER):
            specs.append((f, shape, 0x6E71F000 + 10 * k + workloads.CONFIG5_ROTATION.index(f),
                          workloads.recipe_for(f), 0))
    mix = Mix(specs, "bf16")
    announce("many: Llama-3-8B layer x5 formats")
    assert mix.run() == (0, -1)
    for k, it in enumerate(mix.items):
        single = nq.dequantize_packed(it["fmt"], it["payload"], it["shape"], torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(single.reshape(-1).view(torch.int16), it["out"].view(torch.int16)), (k, it["fmt"])
        nb = it["nel"] // nq.format_query(it["fmt"]).block_values
        ids = np.unique(np.concatenate([[0, nb - 1], np.random.default_rng(k).integers(0, nb, 512)]))
        got = to_numpy(it["out"].reshape(nb, -1)[torch.from_numpy(ids).to("cuda:0")], "bf16").ravel()
        assert compare.same(got, oracle_blocks(it["fmt"], it["p"], ids, "bf16"), "bf16"), (k, it["fmt"])


def test_many_errors_write_nothing():
    specs = [("gguf:q8_0", [4, 64], 1, RECIPE, 0), ("nvfp4", [2, 128], 2, RECIPE, 0)]
    mix = Mix(specs, "f32")
    descs = mix.descs()
    bad = list(descs[1])
    bad[2] -= 1  # length rule
    announce("many: metadata errors")
    st, failed = nq.dequantize_packed_many_raw(descs + [tuple(bad)], 0, torch.cuda.current_stream().cuda_stream)
    assert (st, failed) == (6, 2)
    mis = list(descs[0])
    mis[4] += 2  # f32 output not element-aligned
    st, failed = nq.dequantize_packed_many_raw([descs[0], tuple(mis)], 0, torch.cuda.current_stream().cuda_stream)
    assert (st, failed) == (11, 1)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(mix.buf))


def test_many_on_a_side_stream_and_in_a_graph():
    specs = [(f, [37, 512], 60 + i, RECIPE, 0) for i, f in enumerate(("gguf:q4_k", "gguf:q6_k", "nvfp4",
                                                                       "gguf:q8_0", "gguf:q4_k"))]
    mix = Mix(specs, "bf16")
    s = torch.cuda.Stream()
    announce("many: side stream")
    with torch.cuda.stream(s):
        assert mix.run(stream=s) == (0, -1)
    mix.check("side stream")
    ref = mix.buf.clone()
    g = torch.cuda.CUDAGraph()
    announce("many: graph capture")
    with torch.cuda.graph(g):
        st, failed = nq.dequantize_packed_many_raw(mix.descs(), 2, torch.cuda.current_stream().cuda_stream)
        assert st == 0
    for r in range(3):
        announce(f"many: graph replay {r}")
        for it in mix.items:
            it["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(mix.buf.view(torch.int16), ref.view(torch.int16)), r


def _stream_expected(src, ndst, c):
    """The output nq_measure_stream specifies, from the source chunks (uint32 [n, 4])."""
    nsrc = src.shape[0]
    per_tile = 256 * c
    ntiles = (ndst + per_tile - 1) // per_tile
    out = np.zeros((ndst, 4), dtype=np.uint32)
    for t in range(ntiles):
        lo, hi = t * nsrc // ntiles, (t + 1) * nsrc // ntiles
        acc = np.zeros((256, 4), dtype=np.uint32)
        for k in range(c):
            i = lo + k * 256 + np.arange(256)
            ok = i < hi
            acc[ok] ^= src[i[ok]]
        for k in range(c):
            o = t * per_tile + k * 256 + np.arange(256)
            ok = o < ndst
            v = acc.copy()
            v[:, 0] ^= k
            out[o[ok]] = v[ok]
    return out


@pytest.mark.parametrize("src_chunks,dst_chunks,c,flags", [(1000, 5000, 8, 3), (5000, 5000, 8, 0), (1, 2049, 8, 2),
                                                            (4608, 16384, 2, 2), (7, 7, 1, 1), (3000, 3001, 4, 3),
                                                            (1200, 4000, 1, 0)])
def test_measure_stream_writes_its_pattern(src_chunks, dst_chunks, c, flags):
    rng = np.random.default_rng(src_chunks)
    src = rng.integers(0, 2 ** 32, size=(src_chunks, 4), dtype=np.uint32)
    s = torch.from_numpy(src.view(np.int32)).to("cuda:0")
    d = torch.zeros((dst_chunks + 64, 4), dtype=torch.int32, device="cuda:0")
    announce(f"measure_stream {src_chunks} -> {dst_chunks} c={c} flags={flags}")
    st = nq.measure_stream_raw(s.data_ptr(), 16 * src_chunks, d.data_ptr(), 16 * dst_chunks, c, flags,
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    got = d.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:dst_chunks], _stream_expected(src, dst_chunks, c))
    assert not got[dst_chunks:].any()
