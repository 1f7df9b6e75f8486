"""Pins for the oracle's routing and MoE layer.

Routing is checked against numpy's stable lexicographic sort and scipy's
softmax.  The layer is checked against an explicit composition written here
with torch's SiLU (an independent implementation), against a single-expert FFN
when k = 1, and for invariance under a relabelling of the expert bank."""
import numpy as np
import scipy.special
import torch

import oracle
import workloads


def _bank(E, H, I, seed=0):
    w13 = [workloads.master_weights(2 * I, H, workload=workloads.MOE_LAYER, tensor=workloads.T_W13,
                                    expert=e, seed=seed) for e in range(E)]
    w2 = [workloads.master_weights(H, I, workload=workloads.MOE_LAYER, tensor=workloads.T_W2,
                                   expert=e, seed=seed) for e in range(E)]
    q13 = [oracle.block_quant_fp8(w) for w in w13]
    q2 = [oracle.block_quant_fp8(w) for w in w2]
    return [(a[0], a[1], b[0], b[1]) for a, b in zip(q13, q2)]


def test_route_topk_matches_lexsort_and_softmax():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((6, 64)).astype(np.float32)
    lg[0, [3, 9, 17]] = 2.5          # a three-way tie at the top
    lg[1, :] = 0.0                   # everything tied
    lg[2, 40] = lg[2, 41] = lg[2].max() + 1
    ids, w = oracle.route_topk(lg, 8)
    for m in range(lg.shape[0]):
        order = np.lexsort((np.arange(64), -lg[m].astype(np.float64)))
        assert np.array_equal(ids[m], order[:8])
        assert np.allclose(w[m], scipy.special.softmax(lg[m, order[:8]].astype(np.float64)), rtol=1e-14)
        assert abs(w[m].sum() - 1.0) < 1e-15
    assert list(ids[0, :3]) == [3, 9, 17]
    assert list(ids[1]) == list(range(8))


def _explicit_layer(x_bits, bank, ids, wts):
    qx, sx = oracle.act_quant_fp8(x_bits)
    M, H = x_bits.shape
    out = np.zeros((M, H))
    for m in range(M):
        for j in range(ids.shape[1]):
            q13, s13, q2, s2 = bank[ids[m, j]]
            I = q13.shape[0] // 2
            y13, _ = oracle.gemv_fp8(qx[m:m + 1], sx[m:m + 1], q13, s13)
            g = torch.from_numpy(y13[0, :I])
            u = torch.from_numpy(y13[0, I:])
            h = (torch.nn.functional.silu(g) * u).numpy()
            hb = torch.from_numpy(h).to(torch.bfloat16).float().numpy()      # fp64 -> bf16 via torch
            hq, hs = oracle.block_quant_fp8(hb[None, :])
            y2, _ = oracle.gemv_fp8(hq, hs, q2, s2)
            out[m] += wts[m, j] * y2[0]
    return out


def test_moe_layer_equals_explicit_composition():
    E, H, I, M = 12, 256, 256, 3
    bank = _bank(E, H, I)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=2)
    lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=2)
    r = oracle.moe_layer(x, lambda e: bank[e], logits=lg, top_k=4)
    ids, w = oracle.route_topk(lg, 4)
    assert np.array_equal(r["ids"], ids)
    ref = _explicit_layer(x, bank, ids, w)
    # torch's fp64->bf16 cast may round via fp32; allow a few differing h codes
    assert np.all(np.abs(r["out"] - ref) <= 1e-3 * r["S"])
    assert np.median(np.abs(r["out"] - ref) / r["S"]) < 1e-12


def test_moe_single_expert_reduces_to_ffn():
    E, H, I = 4, 256, 256
    bank = _bank(E, H, I, seed=1)
    x = workloads.activation_bf16(1, H, workload=workloads.MOE_LAYER, seed=3)
    r = oracle.moe_layer(x, lambda e: bank[e], ids=np.array([[2]]), weights=np.array([[1.0]]))
    q13, s13, q2, s2 = bank[2]
    qx, sx = oracle.act_quant_fp8(x)
    y13, _ = oracle.gemv_fp8(qx, sx, q13, s13)
    h = oracle.silu_mul(y13)
    hq, hs = oracle.act_quant_fp8(oracle.bf16_bits(h))
    y2, _ = oracle.gemv_fp8(hq, hs, q2, s2)
    assert np.array_equal(r["out"], y2)
    assert np.array_equal(r["hq"][0, 0], hq[0]) and np.array_equal(r["hs"][0, 0], hs[0])


def test_moe_invariant_under_bank_relabelling():
    E, H, I, M = 10, 256, 256, 2
    bank = _bank(E, H, I, seed=4)
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=4)
    ids = np.array([[1, 7, 3], [7, 0, 9]])
    w = np.array([[0.5, 0.3, 0.2], [0.6, 0.25, 0.15]])
    perm = np.random.default_rng(4).permutation(E)          # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    r0 = oracle.moe_layer(x, lambda e: bank[e], ids=ids, weights=w)
    r1 = oracle.moe_layer(x, lambda e: bank[inv[e]], ids=perm[ids], weights=w)
    assert np.array_equal(r0["out"], r1["out"])


def test_moe_rows_independent_of_batch():
    E, H, I = 8, 256, 256
    bank = _bank(E, H, I, seed=5)
    x = workloads.activation_bf16(3, H, workload=workloads.MOE_LAYER, seed=5)
    lg = workloads.router_logits(3, E, workload=workloads.MOE_LAYER, seed=5)
    r = oracle.moe_layer(x, lambda e: bank[e], logits=lg, top_k=3)
    for m in range(3):
        rm = oracle.moe_layer(x[m:m + 1], lambda e: bank[e], logits=lg[m:m + 1], top_k=3)
        assert np.all(np.abs(rm["out"][0] - r["out"][m]) <= 2.0 ** -45 * r["S"][m])
