"""GPU parity of the standalone quantisers: bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from _helpers import need_gpu, np_bf16_bits_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    need_gpu()
    import quantized_moe_weight_amd as pq
    return pq


@pytest.mark.parametrize("rows,K", [(1, 128), (3, 640), (256, 512), (37, 6144), (4096, 2048)])
def test_quantize_fp8_weights_bit_exact(pq, rows, K):
    import torch
    w = workloads.master_weights(rows, K, workload=workloads.FP8_GEMV_SMALL, seed=rows + K)
    q, s = pq.quantize_fp8(torch.from_numpy(w).cuda())
    qo, so = oracle.block_quant_fp8(w)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_quantize_fp8_every_bf16_pattern(pq):
    """Every finite bf16 value next to a fixed amax, plus zero groups and signed zeros."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = workloads.bf16_bits_to_f32(bits)
    keep = np.isfinite(vals) & (np.abs(vals) < 1000.0)
    bits = bits[keep]
    n = len(bits) // 127 * 127
    grp = bits[:n].reshape(-1, 127)
    amax = workloads.f32_to_bf16_bits(np.full((grp.shape[0], 1), 1000.0, np.float32))
    x = np.concatenate([grp, amax], axis=1).reshape(-1, 128 * 4)          # 4 groups per row
    x = np.concatenate([x, np.zeros((1, 512), np.uint16), np.full((1, 512), 0x8000, np.uint16)], axis=0)
    q, s = pq.quantize_fp8(np_bf16_bits_to_torch(x))
    qo, so = oracle.act_quant_fp8(x)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_quantize_fp8_extreme_ranges(pq):
    import torch
    rng = np.random.default_rng(0)
    rows = []
    for lo, hi in [(-40, -30), (-130, -120), (100, 127), (-5, 5), (-149, -140)]:
        mag = np.exp2(rng.uniform(lo, hi, 128)).astype(np.float32)
        rows.append(mag * rng.choice([-1, 1], 128).astype(np.float32))
    rows.append(np.zeros(128, np.float32))
    w = np.stack(rows).astype(np.float32)
    q, s = pq.quantize_fp8(torch.from_numpy(w).cuda())
    qo, so = oracle.block_quant_fp8(w)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("N,K", [(1, 32), (5, 96), (64, 5120), (333, 1024)])
def test_quantize_q4_bit_exact(pq, N, K):
    import torch
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=N * 7 + K)
    if N > 1:
        w[1, :32] = 0.0                                   # an all-zero group
    p, s = pq.quantize_q4(torch.from_numpy(w).cuda())
    po, so = oracle.q4_quant(w)
    assert np.array_equal(p.cpu().numpy(), po)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), so.view(np.uint16))


def test_quantize_q4_hand_derived_scale_goldens(pq):
    """The library's int4 quantiser on the hand-derived fp16 tie cases (normal,
    subnormal, overflow): every scale equals the fixture's value."""
    import torch
    from test_oracle_quant import q4_golden_rows
    w, exp = q4_golden_rows()
    p, s = pq.quantize_q4(torch.from_numpy(w).cuda())
    got = s.cpu().numpy().view(np.uint16)[:, 0]
    assert np.array_equal(got, exp), [f"0x{g:04x}/0x{e:04x}" for g, e in zip(got, exp)]
    po, _ = oracle.q4_quant(w)
    assert np.array_equal(p.cpu().numpy(), po)
