"""GPU: the batched product without a caller workspace (nq_gemm_q8_1_noalloc).

Its workspace is the library's static device scratch, shared by every call
on a GPU and keeping the last call's contents.  Each call must give the bits
nq_gemm_q8_1 gives with a workspace of its own (the same plan and kernels),
and meet the oracle's criterion on sampled rows; calls follow each other with
smaller shapes, so a call finds the previous call's partials in the scratch.
A shape past the scratch is refused without touching the output.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_nq_amd as nq
import oracle
import synth
from gpu_util import announce, upload
from linear_criterion import check as linear_check

pytestmark = pytest.mark.gpu


def _act(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * 2.0
    x[:, rng.integers(0, K, size=max(1, K // 61))] *= 30.0
    return x.astype(np.float32)


def _run(fmt, N, K, M, seed):
    info = nq.format_query(fmt)
    nb = N * K // info.block_values
    w_np = synth.payload(fmt, nb, seed, synth.binade(-6, -2, False))
    _, xq_np = oracle.quantize_q8_1(_act(M, K, seed + 1))
    w, _keep = upload(w_np)
    xq = torch.from_numpy(np.ascontiguousarray(xq_np)).cuda()
    st, need = nq.gemm_q8_1_workspace(fmt, N, K, M)
    assert st == 0 and 0 < need <= nq.GEMM_SCRATCH_BYTES, (fmt, N, K, M, need)
    announce(f"gemm noalloc {fmt} [{N}, {K}] x {M} (workspace {need} B)")
    ref_dev = nq.gemm_q8_1(fmt, w, N, K, xq)  # the binding gives it a workspace of `need` bytes
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    h = torch.cuda.current_stream().cuda_stream
    assert nq.gemm_q8_1_noalloc_raw(info.id, w.data_ptr(), w_np.size, N, K, xq.data_ptr(), M, y.data_ptr(), h) == 0
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), ref_dev.view(torch.int32)), f"{fmt} [{N}, {K}] x {M}: bits differ"
    got = y.cpu().numpy()
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(N).integers(0, N, size=24)])
    sub = w_np.reshape(N, -1)[rows].ravel()
    ref, env = oracle.gemv_q8_1(fmt, sub, rows.size, K, xq_np, M)
    linear_check(got[:, rows], ref, env, K, f"noalloc {fmt} [{N}, {K}] x {M}")


def test_noalloc_two_calls_in_a_row_second_smaller():
    """K split (partials in the scratch), then a smaller K-split shape."""
    _run("gguf:q4_k", 4096, 14336, 64, 11)
    _run("gguf:q6_k", 1024, 4096, 40, 12)


def test_noalloc_weight_rewritten_once_then_smaller():
    """Above 256 activation rows the weight is rewritten once into the
    scratch too; then a smaller shape that only splits K."""
    _run("gguf:q8_0", 1024, 4096, 300, 21)
    _run("gguf:iq4_xs", 512, 4096, 24, 22)


def test_noalloc_refuses_a_shape_past_the_scratch():
    fmt, N, K, M = "gguf:q4_k", 14336, 4096, 512
    info = nq.format_query(fmt)
    st, need = nq.gemm_q8_1_workspace(fmt, N, K, M)
    assert st == 0 and need > nq.GEMM_SCRATCH_BYTES
    w = torch.zeros(N * K // 256 * 144, dtype=torch.uint8, device="cuda:0")
    xq = torch.zeros(M * K // 32 * 36, dtype=torch.uint8, device="cuda:0")
    y = torch.full((M, N), 5.0, dtype=torch.float32, device="cuda:0")
    announce("gemm noalloc refusal")
    assert nq.gemm_q8_1_noalloc_raw(info.id, w.data_ptr(), w.numel(), N, K, xq.data_ptr(), M, y.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream) == 12
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
