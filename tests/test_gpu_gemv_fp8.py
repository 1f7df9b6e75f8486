"""GPU parity of pq_gemv_fp8 (live FP8 activation quant + block-scaled FP8 GEMV,
K split inside a block, SiLU*up epilogue) against the oracle.  The parameter S
sets PQ_BLOCKS_PER_CU, which moves where rows are cut between waves."""
import os

import numpy as np
import pytest

import oracle
import workloads
from _helpers import (assert_gemv_close, assert_silu_close, bf16_to_np, need_gpu,
                      np_bf16_bits_to_torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


class splitk:
    """Set PQ_BLOCKS_PER_CU (how many blocks share the rows, hence where a row's
    K range is cut between waves) for the duration of a block."""

    def __init__(self, s):
        self.s = s

    def __enter__(self):
        self.old = os.environ.get("PQ_BLOCKS_PER_CU")
        if self.s is not None:
            os.environ["PQ_BLOCKS_PER_CU"] = str(self.s)

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("PQ_BLOCKS_PER_CU", None)
        else:
            os.environ["PQ_BLOCKS_PER_CU"] = self.old


class fp8_path:
    """Force the vector (valu) or the matrix-core (mfma) kernel via PQ_FP8_PATH."""

    def __init__(self, kernel):
        self.kernel = kernel

    def __enter__(self):
        self.old = os.environ.get("PQ_FP8_PATH")
        os.environ["PQ_FP8_PATH"] = self.kernel

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("PQ_FP8_PATH", None)
        else:
            os.environ["PQ_FP8_PATH"] = self.old


def _case(M, K, N, seed, workload=workloads.FP8_GEMV_SMALL):
    import torch
    x = workloads.activation_bf16(M, K, workload=workload, seed=seed)
    w = workloads.master_weights(N, K, workload=workload, seed=seed)
    return x, w, np_bf16_bits_to_torch(x), torch.from_numpy(w).cuda()


def _run(pq, xt, wt, epi, s=None):
    """GPU GEMV on library-quantised weights; returns the oracle's own codes and
    scales (checked equal to the library's) for the reference computation."""
    q, sc = pq.quantize_fp8(wt)
    qo, so = oracle.block_quant_fp8(wt.cpu().numpy())
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(sc.cpu().numpy().view(np.uint32), so.view(np.uint32))
    with splitk(s):
        y, xq, xs = pq.gemv_fp8(xt, q, sc, epi=epi, debug=True)
    return y, xq, xs, qo, so


@pytest.mark.parametrize("M,K,N,S", [
    (1, 512, 256, None),        # the small dense GEMV workload
    (1, 512, 256, 1),
    (2, 640, 37, None),         # 5 blocks: a partial 1 KB chunk, ragged N
    (3, 1152, 100, 3),
    (8, 2048, 96, 4),
    (4, 6144, 300, 2),
])
def test_gemv_fp8_plain(pq, M, K, N, S):
    x, w, xt, wt = _case(M, K, N, seed=M * 100 + K + N)
    y, xq, xs, q, sc = _run(pq, xt, wt, pq.EPI_NONE, S)
    qx, sx = oracle.act_quant_fp8(x)
    assert np.array_equal(xq.cpu().numpy(), qx)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sx.view(np.uint32))
    yo, So = oracle.gemv_fp8(qx, sx, q, sc)
    assert_gemv_close(bf16_to_np(y), yo, So, f"M={M} K={K} N={N} S={S}")


@pytest.mark.parametrize("M,K,N,S", [
    (1, 6144, 4096, None),      # one expert gate_up at batch 1 (gate||up, SiLU*up)
    (1, 6144, 4096, 3),
    (2, 1024, 70, None),
    (5, 768, 64, 2),
])
def test_gemv_fp8_silu(pq, M, K, N, S):
    x, w, xt, wt = _case(M, K, N, seed=M + K + N, workload=workloads.FP8_GATE_UP)
    y, xq, xs, q, sc = _run(pq, xt, wt, pq.EPI_SILU_MUL, S)
    qx, sx = oracle.act_quant_fp8(x)
    assert np.array_equal(xq.cpu().numpy(), qx)
    yo, So = oracle.gemv_fp8(qx, sx, q, sc)
    I = N // 2
    h = oracle.silu_mul(yo, I)
    assert_silu_close(bf16_to_np(y), h, yo[:, :I], yo[:, I:], So[:, :I], So[:, I:], f"M={M} S={S}")


@pytest.mark.parametrize("kernel,M", [("valu", 1), ("mfma", 1), ("mfma", 5)])
def test_gemv_fp8_decodes_every_code(pq, kernel, M):
    """Weight rows hold each of the 256 codes at one position and x is 448 there:
    y[n] = 448 * dq(code_n) exactly (NaN for the two NaN codes).  With M > 1
    the other tokens are zero: their outputs are exactly zero, except NaN on the
    two NaN-code rows (0 * NaN is NaN, as in the dequantise-then-multiply
    definition)."""
    import torch
    K, k0 = 256, 77
    w = np.zeros((256, K), np.uint8)
    w[:, k0] = np.arange(256, dtype=np.uint8)
    sw = np.ones((256, 2), np.float32)
    x = np.zeros((M, K), np.uint16)
    x[0, k0] = workloads.f32_to_bf16_bits(np.array([448.0], np.float32))[0]
    with fp8_path(kernel):
        y = pq.gemv_fp8(np_bf16_bits_to_torch(x), torch.from_numpy(w).cuda(), torch.from_numpy(sw).cuda())
    out = bf16_to_np(y)
    nan_rows = np.isnan(oracle.e4m3_decode(np.arange(256, dtype=np.uint8)))
    assert np.all(np.isnan(out[1:, nan_rows])) and np.all(out[1:, ~nan_rows] == 0)
    got = out[0]
    want = 448.0 * oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_gemv_fp8_rows_bitwise_independent_of_M(pq, kernel):
    """On either kernel a token's outputs do not depend on the other tokens of
    the call (the split of the rows depends on the shape and device only)."""
    import torch
    M, K, N = 6, 2048, 512
    x, w, xt, wt = _case(M, K, N, seed=17)
    q, sc = pq.quantize_fp8(wt)
    with splitk(1), fp8_path(kernel):
        y = pq.gemv_fp8(xt, q, sc, epi=pq.EPI_SILU_MUL)
        for m in range(M):
            ym = pq.gemv_fp8(xt[m:m + 1].contiguous(), q, sc, epi=pq.EPI_SILU_MUL)
            assert torch.equal(ym[0].view(torch.int16), y[m].view(torch.int16))


@pytest.mark.parametrize("M,K,N,epi,S", [
    (4, 6144, 4096, 1, None),   # one expert gate_up, 4 draft tokens
    (8, 6144, 4096, 1, None),
    (8, 6144, 300, 0, None),    # ragged last tile (300 = 18 x 16 + 12)
    (5, 128, 50, 0, None),      # one K block per row: every tile cut between waves or not at all
    (7, 2048, 4000, 0, 2),      # two blocks per CU
    (6, 1152, 70, 1, 3),        # SiLU with a ragged tile, odd K blocks (9)
    (1, 640, 37, 0, None),      # the matrix kernel forced below its default range
    (2, 4096, 1000, 1, None),
    (3, 2560, 129, 0, 1),
])
def test_gemv_fp8_mfma_kernel(pq, M, K, N, epi, S):
    """The matrix-core kernel (the default for M >= 4; forced here for every
    case) against the oracle; the activation codes and scales bit-exact."""
    wl = workloads.FP8_GATE_UP if epi else workloads.FP8_GEMV_SMALL
    x, w, xt, wt = _case(M, K, N, seed=1000 + M * 7 + K + N, workload=wl)
    with fp8_path("mfma"):
        y, xq, xs, q, sc = _run(pq, xt, wt, pq.EPI_SILU_MUL if epi else pq.EPI_NONE, S)
    qx, sx = oracle.act_quant_fp8(x)
    assert np.array_equal(xq.cpu().numpy(), qx)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), sx.view(np.uint32))
    yo, So = oracle.gemv_fp8(qx, sx, q, sc)
    if epi:
        I = N // 2
        h = oracle.silu_mul(yo, I)
        assert_silu_close(bf16_to_np(y), h, yo[:, :I], yo[:, I:], So[:, :I], So[:, I:], f"mfma M={M} N={N}")
    else:
        assert_gemv_close(bf16_to_np(y), yo, So, f"mfma M={M} K={K} N={N} S={S}")


def test_gemv_fp8_mfma_repeat_calls_reset_counters(pq):
    """Back-to-back calls on one workspace (the per-tile arrival counters are
    reset by the last arriver) give identical bits, also across shapes."""
    import torch
    with fp8_path("mfma"):
        x, w, xt, wt = _case(8, 2048, 1000, seed=5)
        q, sc = pq.quantize_fp8(wt)
        y0 = pq.gemv_fp8(xt, q, sc)
        x2, w2, xt2, wt2 = _case(5, 512, 333, seed=6)
        q2, sc2 = pq.quantize_fp8(wt2)
        z0 = pq.gemv_fp8(xt2, q2, sc2)
        for _ in range(10):
            assert torch.equal(pq.gemv_fp8(xt, q, sc).view(torch.int16), y0.view(torch.int16))
            assert torch.equal(pq.gemv_fp8(xt2, q2, sc2).view(torch.int16), z0.view(torch.int16))


def test_gemv_fp8_deterministic_repeats(pq):
    import torch
    x, w, xt, wt = _case(1, 6144, 4096, seed=3, workload=workloads.FP8_GATE_UP)
    q, sc = pq.quantize_fp8(wt)
    for s in (None, 4):
        with splitk(s):
            y0 = pq.gemv_fp8(xt, q, sc, epi=pq.EPI_SILU_MUL)
            for _ in range(20):
                assert torch.equal(pq.gemv_fp8(xt, q, sc, epi=pq.EPI_SILU_MUL).view(torch.int16),
                                   y0.view(torch.int16))


def test_gemv_fp8_zero_inputs_give_zero(pq):
    import torch
    K, N = 512, 64
    x = np.zeros((2, K), np.uint16)
    w = workloads.master_weights(N, K, workload=workloads.FP8_GEMV_SMALL, seed=1)
    q, sc = pq.quantize_fp8(torch.from_numpy(w).cuda())
    y = pq.gemv_fp8(np_bf16_bits_to_torch(x), q, sc)
    assert torch.all(y == 0)


def test_gemv_fp8_rejects_bad_shapes(pq):
    import torch
    x = torch.zeros((1, 100), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4, 100), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    with pytest.raises((pq.PqError, ValueError)):
        pq.gemv_fp8(x, w, s)
    x = torch.zeros((9, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(pq.PqError):
        pq.gemv_fp8(x, w, s)


@pytest.mark.parametrize("M", [1, 8])
def test_gemv_fp8_lm_head_sampled_rows(pq, M):
    """LM-head GEMV at full vocabulary width (K=6144, N=151552, one launch): the
    master weights are drawn on the device, quantised by the library, and a sample
    of output rows (the first and last 128, plus 1536 drawn at random) is checked
    against the oracle, which quantises just those rows' master weights (the
    1x128 blocks of one row do not depend on any other row)."""
    import torch
    K, N = 6144, workloads.LM_HEAD_V
    x = workloads.activation_bf16(M, K, workload=workloads.LM_HEAD, seed=M)
    xt = np_bf16_bits_to_torch(x)
    wt = workloads.master_weights_torch(N, K, workload=workloads.LM_HEAD, seed=M)
    q, sc = pq.quantize_fp8(wt)
    y, xq, xs = pq.gemv_fp8(xt, q, sc, debug=True)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(N - 128, N),
                                     rng.choice(N, 1536, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    w_rows = wt.index_select(0, ridx).cpu().numpy()
    del wt
    qo, so = oracle.block_quant_fp8(w_rows)
    assert np.array_equal(q.index_select(0, ridx).cpu().numpy(), qo)
    assert np.array_equal(sc.index_select(0, ridx).cpu().numpy().view(np.uint32), so.view(np.uint32))
    qx, sx = oracle.act_quant_fp8(x)
    assert np.array_equal(xq.cpu().numpy(), qx)
    yo, So = oracle.gemv_fp8(qx, sx, qo, so)
    got = bf16_to_np(y)[:, rows]
    assert_gemv_close(got, yo, So, f"lm_head M={M} rows={len(rows)}")
