"""Helpers for GPU tests: upload, decode through the C ABI, download."""
import concurrent.futures
import os
import sys

import numpy as np
import torch

import block_quantized_weight_nq_amd as nq
import oracle

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}
NP_VIEW = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}


def announce(msg):
    """Name the case on the real stderr (not pytest's capture) before a GPU step."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def to_numpy(t, dtype):
    t = t.detach().cpu()
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def upload(payload_np, pay_off=0, device="cuda:0"):
    """A rank-1 uint8 CUDA tensor holding payload_np at byte offset pay_off of its allocation."""
    n = payload_np.size
    buf = torch.zeros(n + pay_off + 64, dtype=torch.uint8, device=device)
    if n:
        buf[pay_off:pay_off + n].copy_(torch.from_numpy(np.ascontiguousarray(payload_np)))
    return buf[pay_off:pay_off + n], buf


def decode(fmt, payload_np, shape, dtype, pay_off=0, out_off=0, stream=None):
    """Decode on cuda:0; returns (values as numpy, out allocation, output view)."""
    payload, _keep = upload(payload_np, pay_off)
    nel = int(np.prod(shape)) if len(shape) else 1
    obuf = torch.full((nel + out_off + 8,), float("nan"), dtype=TORCH_DT[dtype], device="cuda:0")
    out = obuf[out_off:out_off + nel]
    nq.dequantize_packed(fmt, payload, shape, TORCH_DT[dtype], out=out, stream=stream)
    torch.cuda.synchronize()
    return to_numpy(out, dtype), obuf, out


def oracle_blocks(fmt, payload_np, block_ids, dtype):
    """Oracle values of selected blocks of a payload, converted to dtype."""
    _, B, S, T = oracle.info(fmt)
    d_w = 0.0
    if T == 4:
        d_w = float(payload_np[-4:].copy().view("<f4")[0])
    idx = np.asarray(block_ids, dtype=np.int64)
    rows = payload_np[: (payload_np.size - T)].reshape(-1, S)[idx]
    f32 = oracle.decode_blocks_f32(fmt, rows.ravel(), d_w)
    return oracle.convert(f32, dtype) if dtype != "f32" else f32


def oracle_threads():
    """Host threads for fanned-out oracle decodes: the cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_decode_parallel(fmt, payload_np, nblocks, dtype, threads=None):
    """The oracle's decode of a whole payload, its blocks split over host threads
    (blocks decode independently; each chunk carries the format's trailer).
    The first block is decoded on this thread first, so the oracle's lazily
    built codebooks exist before the threads start."""
    _, B, S, T = oracle.info(fmt)
    threads = threads or oracle_threads()
    trailer = payload_np[nblocks * S:] if T else None

    def part(b0, b1):
        q = payload_np[b0 * S:b1 * S]
        if T:
            q = np.concatenate([q, trailer])
        return oracle.decode(fmt, q, [(b1 - b0) * B], dtype)

    if nblocks == 0:
        return part(0, 0)
    part(0, 1)
    n = min(nblocks, threads * 4)
    edges = [nblocks * k // n for k in range(n + 1)]
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda k: part(edges[k], edges[k + 1]), range(n)))
    return np.concatenate(parts)
