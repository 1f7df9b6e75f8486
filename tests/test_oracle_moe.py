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


def test_router_logits_exact_rational_brute_force():
    """The router's fp64 logits equal the exact rational dot products of the
    bf16 inputs (every bf16 value is a dyadic rational; the sums of 64 of them
    are exact in fp64 here because the magnitudes are bounded)."""
    from fractions import Fraction
    rng = np.random.default_rng(9)
    M, E, H = 2, 5, 64
    x = workloads.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    wr = workloads.f32_to_bf16_bits((0.05 * rng.standard_normal((E, H))).astype(np.float32))
    lg = oracle.router_logits(x, wr)
    xv = workloads.bf16_bits_to_f32(x).astype(np.float64)
    wv = workloads.bf16_bits_to_f32(wr).astype(np.float64)
    for m in range(M):
        for e in range(E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[m], wv[e]))
            assert abs(Fraction(float(lg[m, e])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_router_logits_one_hot_rows_select_inputs():
    """A router row that is 1.0 at position k and 0 elsewhere gives x[m, k]
    exactly; a row of 2.0 gives twice the sum (closed forms)."""
    rng = np.random.default_rng(10)
    M, H = 3, 256
    x = workloads.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    one = workloads.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    two = workloads.f32_to_bf16_bits(np.array([2.0], np.float32))[0]
    wr = np.zeros((4, H), np.uint16)
    for e, k in enumerate([0, 7, 100, 255]):
        wr[e, k] = one
    lg = oracle.router_logits(x, wr)
    xv = workloads.bf16_bits_to_f32(x).astype(np.float64)
    assert np.array_equal(lg, xv[:, [0, 7, 100, 255]])
    lg2 = oracle.router_logits(x, np.full((1, H), two, np.uint16))
    assert np.allclose(lg2[:, 0], 2.0 * xv.sum(axis=1), rtol=0, atol=1e-12)


def test_router_logits_match_torch_float64():
    """Against torch's own bf16 -> fp64 conversion and fp64 matmul."""
    rng = np.random.default_rng(11)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((4, 512)).astype(np.float32))
    wr = workloads.f32_to_bf16_bits((0.02 * rng.standard_normal((32, 512))).astype(np.float32))
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()
    tw = torch.from_numpy(wr.view(np.int16)).view(torch.bfloat16).double()
    ref = (tx @ tw.T).numpy()
    assert np.allclose(oracle.router_logits(x, wr), ref, rtol=1e-13, atol=1e-13)


def test_shared_expert_is_a_weight_one_slot_after_the_routed_slots():
    """The layer with a shared expert equals the layer without it whose every
    token gets one more slot, after its routed slots, on the shared expert with
    weight 1 (a decomposition into the already-pinned routed layer)."""
    E, H, I, M, k = 9, 256, 256, 3, 3
    bank = _bank(E + 1, H, I, seed=7)                 # expert E plays the shared one
    x = workloads.activation_bf16(M, H, workload=workloads.MOE_LAYER, seed=7)
    lg = workloads.router_logits(M, E, workload=workloads.MOE_LAYER, seed=7)
    ids, w = oracle.route_topk(lg, k)
    r = oracle.moe_layer(x, lambda e: bank[e], logits=lg, top_k=k, shared=bank[E])
    ids2 = np.concatenate([ids, np.full((M, 1), E)], axis=1)
    w2 = np.concatenate([w, np.ones((M, 1))], axis=1)
    r2 = oracle.moe_layer(x, lambda e: bank[e], ids=ids2, weights=w2)
    assert np.array_equal(r["out"], r2["out"])
    assert np.array_equal(r["S"], r2["S"])
    assert np.array_equal(r["sh_hq"], r2["hq"][:, k]) and np.array_equal(r["sh_hs"], r2["hs"][:, k])
    assert np.array_equal(r["sh_h_bits"], r2["h_bits"][:, k])
    # and against the explicit torch-SiLU composition
    ref = _explicit_layer(x, bank, ids2, w2)
    assert np.all(np.abs(r["out"] - ref) <= 1e-3 * r["S"])
