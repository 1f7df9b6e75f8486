"""GPU parity of moe_decode_layer_noalloc (the layer with its workspace in the
library's static per-GPU scratch) against the workspace entry point
moe_decode_layer_ex, through the C ABI: two calls in a row, the second with a
smaller input, on both layer kernels, with and without the router GEMV and a
shared expert in the launch.  The two entry points run the same kernels on
the same inputs, so their outputs must be bitwise equal; the first call is
also checked against the oracle.  Device-side errors come back through the
status pointer, one call at a time."""
import os

import numpy as np
import pytest

import oracle
import workloads
from _helpers import assert_gemv_close, bf16_to_np, need_gpu, np_bf16_bits_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


class moe_path:
    def __init__(self, p):
        self.p = p

    def __enter__(self):
        self.old = os.environ.get("PQ_MOE_PATH")
        os.environ["PQ_MOE_PATH"] = self.p

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop("PQ_MOE_PATH", None)
        else:
            os.environ["PQ_MOE_PATH"] = self.old


def _same(a, b):
    import torch
    return torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                       b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32))


@pytest.mark.parametrize("path", ["barrier", "stream"])
def test_noalloc_equals_workspace_entry_point(pq, path):
    import torch
    from test_gpu_moe import Bank
    E, H, I, k = 24, 1024, 512, 8
    bank = Bank(pq, E, H, I, seed=80)
    for step, M in enumerate((6, 1)):            # the second call is smaller
        x = workloads.activation_bf16(M, H, workload=workloads.MOE_VERIFY, seed=80 + M)
        lg = workloads.verify_logits(M, E, seed=80 + M)
        bank.fill(oracle.route_topk(lg, k)[0])
        xt, lt = np_bf16_bits_to_torch(x), torch.from_numpy(lg).cuda()
        with moe_path(path):
            ref = pq.moe_decode_layer(xt, bank.w13, bank.s13, bank.w2, bank.s2, logits=lt, top_k=k)
            assert pq.workspace_check() == 0
            got = pq.moe_decode_layer_noalloc(xt, bank.w13, bank.s13, bank.w2, bank.s2, logits=lt, top_k=k)
        torch.cuda.synchronize()
        assert int(got["status"][0]) == 0
        assert _same(got["out"], ref["out"]), f"call {step} (M={M}): outputs differ from the workspace entry point"
        assert torch.equal(got["topk_ids"], ref["topk_ids"]) and _same(got["topk_w"], ref["topk_w"])
        if step == 0:
            o = oracle.moe_layer(x, bank.expert, logits=lg, top_k=k)
            assert_gemv_close(bf16_to_np(got["out"]), o["out"], o["S"], f"noalloc M={M}")


@pytest.mark.parametrize("path", ["barrier", "stream"])
def test_noalloc_with_router_and_shared_expert(pq, path):
    import torch
    from test_gpu_moe import Bank
    E, H, I, k = 32, 1024, 256, 8
    bank = Bank(pq, E, H, I, seed=81)
    sh = bank.shared()
    bank.fill(range(E))
    wr = workloads.router_weights_bf16(E, H, seed=81)
    wrt = np_bf16_bits_to_torch(wr)
    for M in (4, 2):
        x = workloads.activation_bf16(M, H, workload=workloads.MOE_VERIFY, seed=90 + M)
        xt = np_bf16_bits_to_torch(x)
        with moe_path(path):
            ref = pq.moe_decode_layer(xt, bank.w13, bank.s13, bank.w2, bank.s2, router_w=wrt, top_k=k, shared=sh)
            assert pq.workspace_check() == 0
            got = pq.moe_decode_layer_noalloc(xt, bank.w13, bank.s13, bank.w2, bank.s2, router_w=wrt, top_k=k,
                                              shared=sh)
        torch.cuda.synchronize()
        assert int(got["status"][0]) == 0
        assert _same(got["logits"], ref["logits"])
        assert torch.equal(got["topk_ids"], ref["topk_ids"])
        assert _same(got["out"], ref["out"]), f"M={M}: outputs differ from the workspace entry point"


def test_noalloc_reports_each_calls_status(pq):
    """A bad expert id given as input is reported through the status pointer of
    that call; the next call reports PQ_OK and is correct."""
    import torch
    from test_gpu_moe import Bank
    E, H, I = 8, 256, 128
    bank = Bank(pq, E, H, I, seed=82)
    bank.fill(range(E))
    x = torch.zeros((1, H), dtype=torch.bfloat16, device="cuda")
    bad = pq.moe_decode_layer_noalloc(x, bank.w13, bank.s13, bank.w2, bank.s2,
                                      topk_ids=torch.tensor([[1, 99]], dtype=torch.int32, device="cuda"),
                                      topk_w=torch.tensor([[0.5, 0.5]], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert int(bad["status"][0]) == -8
    xb = workloads.activation_bf16(1, H, workload=workloads.MOE_LAYER, seed=82)
    ids = np.array([[3, 5]], np.int32)
    w = np.array([[0.75, 0.25]], np.float32)
    good = pq.moe_decode_layer_noalloc(np_bf16_bits_to_torch(xb), bank.w13, bank.s13, bank.w2, bank.s2,
                                       topk_ids=torch.from_numpy(ids).cuda(), topk_w=torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert int(good["status"][0]) == 0
    o = oracle.moe_layer(xb, bank.expert, ids=ids, weights=w.astype(np.float64))
    assert_gemv_close(bf16_to_np(good["out"]), o["out"], o["S"], "noalloc after a bad call")
