"""GPU parity of pq_gemm_fp8 (prefill / large-M block-scaled FP8 GEMM on the
matrix cores, activation quantised live in a first launch) against the oracle.

Expected values come from the oracle on the same seeded inputs: the weights
are quantised by the library and by the oracle and checked equal first; the
activation codes and scales the GEMM used are read back from the workspace and
checked bit-exact against the oracle's.  Large shapes compare a sample of
tokens (all their outputs) computed one by one by the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from _helpers import assert_gemv_close, assert_silu_close, bf16_to_np, need_gpu, np_bf16_bits_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


def _weights(pq, N, K, seed, workload):
    import torch
    w = workloads.master_weights(N, K, workload=workload, seed=seed)
    q, sc = pq.quantize_fp8(torch.from_numpy(w).cuda())
    qo, so = oracle.block_quant_fp8(w)
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(sc.cpu().numpy().view(np.uint32), so.view(np.uint32))
    return q, sc, qo, so


def _compare(y, x, xq, xs, qo, so, epi, rows, what):
    qx, sx = oracle.act_quant_fp8(x[rows])
    assert np.array_equal(xq.cpu().numpy()[rows], qx)
    assert np.array_equal(xs.cpu().numpy()[rows].view(np.uint32), sx.view(np.uint32))
    yo, So = oracle.gemv_fp8(qx, sx, qo, so)
    got = bf16_to_np(y)[rows]
    if epi:
        I = qo.shape[0] // 2
        h = oracle.silu_mul(yo, I)
        return assert_silu_close(got, h, yo[:, :I], yo[:, I:], So[:, :I], So[:, I:], what)
    return assert_gemv_close(got, yo, So, what)


@pytest.mark.parametrize("M,K,N,epi", [
    (1, 128, 64, 0),           # one token, one K block, half a tile
    (17, 640, 200, 0),         # ragged token and weight tiles, 5 K blocks
    (128, 2048, 256, 0),       # whole tiles
    (300, 1024, 1000, 1),      # SiLU*up with ragged output tiles
    (129, 256, 130, 1),        # 65 outputs: one column past a 64-wide tile
    (513, 768, 2000, 0),       # more tiles than CUs
])
def test_gemm_fp8_against_oracle(pq, M, K, N, epi):
    wl = workloads.FP8_GATE_UP if epi else workloads.FP8_GEMV_SMALL
    x = workloads.activation_bf16(M, K, workload=wl, seed=M + K + N)
    q, sc, qo, so = _weights(pq, N, K, seed=M + N, workload=wl)
    y, xq, xs = pq.gemm_fp8(np_bf16_bits_to_torch(x), q, sc, epi=epi, debug=True)
    _compare(y, x, xq, xs, qo, so, epi, np.arange(M), f"M={M} K={K} N={N} epi={epi}")


def test_gemm_fp8_prefill_gate_up_sampled_tokens(pq):
    """One expert's gate_up over a 2048-token prefill chunk (K=6144, N=2x2048,
    SiLU*up): 48 sampled tokens, every output of each."""
    M, K, N = 2048, 6144, 4096
    x = workloads.activation_bf16(M, K, workload=workloads.FP8_GATE_UP, seed=7)
    q, sc, qo, so = _weights(pq, N, K, seed=7, workload=workloads.FP8_GATE_UP)
    y, xq, xs = pq.gemm_fp8(np_bf16_bits_to_torch(x), q, sc, epi=pq.EPI_SILU_MUL, debug=True)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, M - 1], np.random.default_rng(7).choice(M, 43, replace=False)]))
    _compare(y, x, xq, xs, qo, so, 1, rows, "prefill gate_up")


def test_gemm_fp8_rows_independent_of_M(pq):
    """A token's outputs do not depend on the other tokens of the call."""
    import torch
    K, N = 1024, 384
    x = workloads.activation_bf16(200, K, workload=workloads.FP8_GEMV_SMALL, seed=3)
    q, sc, _, _ = _weights(pq, N, K, seed=3, workload=workloads.FP8_GEMV_SMALL)
    xt = np_bf16_bits_to_torch(x)
    y = pq.gemm_fp8(xt, q, sc)
    for m in (0, 77, 199):
        ym = pq.gemm_fp8(xt[m:m + 1].contiguous(), q, sc)
        assert torch.equal(ym[0].view(torch.int16), y[m].view(torch.int16))
    y2 = pq.gemm_fp8(xt[50:180].contiguous(), q, sc)
    assert torch.equal(y2.view(torch.int16), y[50:180].view(torch.int16))


def test_gemm_fp8_leaves_shared_workspace_state(pq):
    """The GEMM's scratch lies in the data region of the shared workspace: the
    counters and the zero-between-calls region the other entry points rely on
    stay zero."""
    import torch
    M, K, N = 1024, 2048, 256
    x = workloads.activation_bf16(M, K, workload=workloads.FP8_GEMV_SMALL, seed=9)
    q, sc, _, _ = _weights(pq, N, K, seed=9, workload=workloads.FP8_GEMV_SMALL)
    pq.gemm_fp8(np_bf16_bits_to_torch(x), q, sc)
    ws, _ = pq._workspace(1)
    torch.cuda.synchronize()
    assert pq.workspace_check() == 0
    assert int(torch.count_nonzero(ws[256:pq.WS_DATA_OFF])) == 0


def test_gemm_fp8_prequant_equals_the_fused_call(pq):
    """The GEMM on the activation quantised beforehand (by the library's own
    quantiser) gives the bits of the call that quantises it itself."""
    import torch
    M, K, N = 333, 1536, 700
    x = workloads.activation_bf16(M, K, workload=workloads.FP8_GATE_UP, seed=12)
    q, sc, _, _ = _weights(pq, N, K, seed=12, workload=workloads.FP8_GATE_UP)
    xt = np_bf16_bits_to_torch(x)
    for epi in (pq.EPI_NONE, pq.EPI_SILU_MUL):
        y = pq.gemm_fp8(xt, q, sc, epi=epi)
        xq, xs = pq.quantize_fp8(xt)
        y2 = pq.gemm_fp8_prequant(xq, xs, q, sc, epi=epi)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_gemm_fp8_rejects_bad_shapes(pq):
    import torch
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 100), dtype=torch.uint8, device="cuda")
    s = torch.zeros((8, 0), dtype=torch.float32, device="cuda")
    with pytest.raises((pq.PqError, ValueError)):
        pq.gemm_fp8(x, w, s)
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((7, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones((7, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(pq.PqError):
        pq.gemm_fp8(x, w, s, epi=pq.EPI_SILU_MUL)
