"""Pins for the traffic closed forms: the figures the pages print
(tests/golden/sionic_traffic_figures.txt) and hand-counted byte totals."""
import os

import numpy as np

import oracle
from oracle import traffic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sionic_traffic_figures.txt")


def _figures():
    out = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, val, dec = line.split()
        out[name] = (float(val), int(dec))
    return out


def _agrees(computed, printed):
    val, dec = printed
    return abs(computed - val) <= 0.5 * 10.0 ** -dec + 1e-12


def test_mtp_traffic_table():
    f = _figures()
    per_fwd = f["bytes_per_forward_gb"][0]
    assert _agrees(traffic.per_accepted_token(per_fwd, 3.5), f["traffic_L3.5_gb"])
    assert _agrees(traffic.per_accepted_token(per_fwd, 10.0), f["traffic_L10_gb"])
    assert traffic.per_accepted_token(per_fwd, 1.0) == per_fwd


def test_bandwidth_floor_and_fractions():
    f = _figures()
    peak = f["hbm_peak_tb_s"][0] * 1e12
    floor_ms = traffic.bandwidth_floor_seconds(f["bytes_per_forward_gb"][0] * 1e9, peak) * 1e3
    assert _agrees(floor_ms, f["floor_ms"])
    for bw, pct in (("gemm_effective_tb_s", "gemm_effective_pct"), ("hmma_tb_s", "hmma_pct"),
                    ("tmem_tb_s", "tmem_pct")):
        assert _agrees(100 * traffic.fraction_of_peak(f[bw][0] * 1e12, peak), f[pct])
    assert _agrees(f["tmem_tb_s"][0] / f["hmma_tb_s"][0], f["tmem_speedup"])


def test_hand_counted_bytes():
    # gate_up 4096x6144 codes + 4096x48 fp32 scales; down 6144x2048 + 6144x16 scales
    assert traffic.fp8_weight_bytes(4096, 6144) == 4096 * 6144 + 4096 * 48 * 4 == 25_952_256
    assert traffic.fp8_weight_bytes(6144, 2048) == 12_976_128
    assert traffic.expert_bytes(6144, 2048) == 38_928_384
    assert traffic.moe_call_bytes(1, 8, 6144, 2048, 256) == 8 * 38_928_384 + 2 * 6144 * 2 + 4 * 256
    assert traffic.fp8_linear_bytes(1, 512, 256) == 131072 + 4096 + 1024 + 512 == 136_704
    assert traffic.fp8_linear_bytes(1, 6144, 4096, silu_mul=True) == 25_952_256 + 12288 + 4096
    # int4 g32: K/2 bytes of nibbles + 2 bytes of fp16 scale per 32 weights (4.5 bits per weight)
    assert traffic.q4_weight_bytes(5120, 5120) * 8 / (5120 * 5120) == 4.5
    assert traffic.q4_linear_bytes(1, 5120, 5120) == 14_745_600 + 10240 + 10240


def test_union_bounds():
    rng = np.random.default_rng(0)
    for M in (1, 2, 4, 8):
        ids, _ = oracle.route_topk(rng.standard_normal((M, 256)).astype(np.float32), 8)
        u = len(oracle.union_of_experts(ids))
        assert 8 <= u <= min(8 * M, 256)
        if M == 1:
            assert u == 8
