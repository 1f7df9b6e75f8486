"""One workspace shared by every entry point (the binding keeps one per stream).

The counter region [256 B, 64 KB) and the zeroed exchange region
[64 KB, 64 KB + 2 MB) must be all zero after every call, whatever the entry
point: the matrix-core GEMVs use the counter words as tile arrival counts and
the layer kernels use them as release flags, so a word left non-zero by one
would corrupt the next.  These tests alternate layer calls on both layer
kernels with matrix-core FP8 and int4 GEMVs whose row tiles are cut between
waves (so their counters are live) on the same workspace, check the regions
after each call, and check every result against the oracle.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from _helpers import assert_gemv_close, bf16_to_np, need_gpu, np_bf16_bits_to_torch

pytestmark = pytest.mark.gpu

COUNTERS = slice(256, 65536)
ZEROED = slice(65536, 65536 + (2 << 20))


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


class env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _ws(pq):
    import torch
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    return pq._WS[key]


def _assert_regions_zero(pq, what):
    import torch
    torch.cuda.synchronize()
    ws = _ws(pq)
    c = ws[COUNTERS].cpu().numpy()
    z = ws[ZEROED].cpu().numpy()
    assert not c.any(), f"after {what}: counter words left non-zero at byte offsets {(np.flatnonzero(c)[:8] + 256).tolist()}"
    assert not z.any(), f"after {what}: exchange region left non-zero"


def _fp8_case(pq, M, K, N, seed):
    import torch
    x = workloads.activation_bf16(M, K, workload=workloads.FP8_GEMV_SMALL, seed=seed)
    w = workloads.master_weights(N, K, workload=workloads.FP8_GEMV_SMALL, seed=seed)
    q, s = pq.quantize_fp8(torch.from_numpy(w).cuda())
    qo, so = oracle.block_quant_fp8(w)
    assert np.array_equal(q.cpu().numpy(), qo)
    qx, sx = oracle.act_quant_fp8(x)
    yo, So = oracle.gemv_fp8(qx, sx, qo, so)
    return np_bf16_bits_to_torch(x), q, s, yo, So


def _q4_case(pq, M, K, N, seed):
    import torch
    x = workloads.activation_bf16(M, K, workload=workloads.Q4_STACK, seed=seed, outliers=0)
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=seed)
    p, s = oracle.q4_quant(w)
    yo, So = oracle.gemv_q4(x, p, s)
    return (np_bf16_bits_to_torch(x), torch.from_numpy(p).cuda(),
            torch.from_numpy(s.view(np.int16)).view(torch.float16).cuda(), yo, So)


def _layer_case(pq, seed):
    import torch
    from test_gpu_moe import Bank
    M, E, H, I, k = 2, 16, 512, 256, 4
    bank = Bank(pq, E, H, I, seed=seed)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=seed)
    lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=seed)
    bank.fill(oracle.route_topk(lg, k)[0])
    ref = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
    return bank, np_bf16_bits_to_torch(x), torch.from_numpy(lg).cuda(), k, ref


def test_layer_calls_and_matrix_gemvs_share_one_workspace(pq):
    # 16384 x 1024 FP8 at M = 4: 1024 tiles of 16 rows over 2048 waves, every
    # tile cut between two waves; int4 8192 x 1024 at M = 5: 512 tiles
    fx, fq, fs, fyo, fSo = _fp8_case(pq, 4, 1024, 16384, seed=31)
    qx, qp, qs, qyo, qSo = _q4_case(pq, 5, 1024, 8192, seed=32)
    bank, lx, llg, k, lref = _layer_case(pq, seed=33)

    def fp8():
        with env(PQ_FP8_PATH="mfma"):
            y = pq.gemv_fp8(fx, fq, fs)
        assert_gemv_close(bf16_to_np(y), fyo, fSo, "FP8 matrix-core GEMV")
        _assert_regions_zero(pq, "FP8 matrix-core GEMV")

    def q4():
        with env(PQ_Q4_PATH="mfma"):
            y = pq.gemv_q4(qx, qp, qs)
        assert_gemv_close(bf16_to_np(y), qyo, qSo, "int4 matrix-core GEMV")
        _assert_regions_zero(pq, "int4 matrix-core GEMV")

    def layer(path):
        with env(PQ_MOE_PATH=path):
            r = pq.moe_decode_layer(lx, bank.w13, bank.s13, bank.w2, bank.s2, logits=llg, top_k=k)
        assert pq.workspace_check() == 0
        assert_gemv_close(bf16_to_np(r["out"]), lref["out"], lref["S"], f"layer ({path})")
        _assert_regions_zero(pq, f"layer call ({path} kernel)")

    fp8()                     # sizes the stream's workspace for the largest user
    q4()
    ws0 = _ws(pq)
    for _ in range(3):
        layer("barrier")
        fp8()
        q4()
        layer("stream")
        q4()
        fp8()
    assert _ws(pq) is ws0, "the calls did not share one workspace"
