"""Pins for the oracle's linear layers (FP8 GEMV, int4 GEMV, SiLU*up epilogue).

Expected values: exact rational brute force on tiny shapes (decoding through
torch's float8 tables, not the oracle's), special cases that reduce to an
integer matrix product, a one-hot weight row that must return the dequantised
activation, and invariants (row independence of M, split-K additivity,
power-of-two scaling).  Shapes are non-square so that a transposed operand or
a swapped index fails.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads


def _t_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _fraction_gemv_fp8(qx, sx, qw, sw):
    xd, wd = _t_decode(qx), _t_decode(qw)
    M, K = qx.shape
    N = qw.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // 128):
                blk = Fraction(0)
                for k in range(128 * b, 128 * (b + 1)):
                    blk += Fraction(float(xd[m, k])) * Fraction(float(wd[n, k]))
                acc += Fraction(float(sx[m, b])) * Fraction(float(sw[n, b])) * blk
            y[m][n] = acc
    return y


@pytest.mark.parametrize("M,K,N", [(1, 128, 3), (2, 256, 5)])
def test_gemv_fp8_matches_exact_rational(M, K, N):
    x = workloads.activation_bf16(M, K, workload=workloads.FP8_GEMV_SMALL, seed=11)
    w = workloads.master_weights(N, K, workload=workloads.FP8_GEMV_SMALL, seed=11)
    qx, sx = oracle.act_quant_fp8(x)
    qw, sw = oracle.block_quant_fp8(w)
    y, S = oracle.gemv_fp8(qx, sx, qw, sw)
    exact = _fraction_gemv_fp8(qx, sx, qw, sw)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - exact[m][n]) <= Fraction(2.0 ** -50) * Fraction(float(S[m, n]))


def test_gemv_fp8_unit_scales_reduce_to_decoded_matmul():
    rng = np.random.default_rng(2)
    qx = rng.integers(0, 0x7E, (3, 256)).astype(np.uint8)
    qw = rng.integers(0, 0x7E, (7, 256)).astype(np.uint8)
    qx[qx == 0x7F] = 0
    one = lambda r: np.ones((r, 2), np.float32)   # noqa: E731
    y, _ = oracle.gemv_fp8(qx, one(3), qw, one(7))
    xd, wd = _t_decode(qx), _t_decode(qw)
    # integer matmul in units of 2^-18 is exact
    xi = np.rint(xd * 2 ** 9).astype(np.int64)
    wi = np.rint(wd * 2 ** 9).astype(np.int64)
    assert np.array_equal(xi / 2 ** 9, xd) and np.array_equal(wi / 2 ** 9, wd)
    assert np.array_equal(y, (xi @ wi.T) / 2.0 ** 18)


def test_gemv_fp8_one_hot_row_returns_dequantised_activation():
    x = workloads.activation_bf16(2, 384, workload=workloads.FP8_GEMV_SMALL, seed=4)
    qx, sx = oracle.act_quant_fp8(x)
    N, K = 5, 384
    qw = np.zeros((N, K), np.uint8)
    sw = np.ones((N, K // 128), np.float32)
    picks = [0, 127, 128, 300, 383]
    for n, k in enumerate(picks):
        qw[n, k] = 0x38                              # 1.0
    y, _ = oracle.gemv_fp8(qx, sx, qw, sw)
    xd = _t_decode(qx)
    for n, k in enumerate(picks):
        assert np.array_equal(y[:, n], xd[:, k] * sx[:, k // 128].astype(np.float64))


def test_gemv_fp8_invariants():
    M, K, N = 4, 512, 6
    x = workloads.activation_bf16(M, K, workload=workloads.FP8_GEMV_SMALL, seed=8)
    w = workloads.master_weights(N, K, workload=workloads.FP8_GEMV_SMALL, seed=8)
    qx, sx = oracle.act_quant_fp8(x)
    qw, sw = oracle.block_quant_fp8(w)
    y, S = oracle.gemv_fp8(qx, sx, qw, sw)
    tol = 2.0 ** -48 * S
    # each row independent of M
    for m in range(M):
        ym, _ = oracle.gemv_fp8(qx[m:m + 1], sx[m:m + 1], qw, sw)
        assert np.all(np.abs(ym[0] - y[m]) <= tol[m])
    # split-K: the sum over K ranges (multiples of 128) equals the unsplit result
    parts = [(0, 128), (128, 384), (384, 512)]
    ys = sum(oracle.gemv_fp8(qx[:, a:b], sx[:, a // 128:b // 128], qw[:, a:b], sw[:, a // 128:b // 128])[0]
             for a, b in parts)
    assert np.all(np.abs(ys - y) <= tol)
    # scaling the master weights by 2^j scales y by 2^j exactly
    qw3, sw3 = oracle.block_quant_fp8(w * np.float32(8.0))
    y3, _ = oracle.gemv_fp8(qx, sx, qw3, sw3)
    assert np.array_equal(y3, 8.0 * y)
    # all-zero activations or weights give exactly zero
    z, _ = oracle.gemv_fp8(np.zeros_like(qx), np.ones_like(sx), qw, sw)
    assert np.all(z == 0)


def test_silu_mul_against_scipy_and_special_values():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((2, 64)) * 5
    u = rng.standard_normal((2, 64))
    h = oracle.silu_mul(np.concatenate([g, u], axis=1))
    ref = g * scipy.special.expit(g) * u
    assert np.allclose(h, ref, rtol=1e-14, atol=0)
    z = oracle.silu_mul(np.array([[0.0, 50.0, -800.0, 2.0, 3.0, 4.0]]))
    assert z[0, 0] == 0.0
    assert abs(z[0, 1] - 50.0 * 3.0) <= 1e-12 * 150
    assert z[0, 2] == 0.0
    # gate rows come first: swapping halves changes the result
    hs = oracle.silu_mul(np.concatenate([u, g], axis=1))
    assert not np.allclose(hs, h)


def test_gemv_q4_unit_scales_reduce_to_integer_matmul():
    rng = np.random.default_rng(5)
    M, K, N = 3, 96, 7
    q = rng.integers(-8, 8, (N, K))
    xi = rng.integers(-50, 50, (M, K))
    x_bits = workloads.f32_to_bf16_bits(xi.astype(np.float32))
    packed = oracle.q4_pack(q)
    s16 = np.ones((N, K // 32), np.float16)
    y, S = oracle.gemv_q4(x_bits, packed, s16)
    assert np.array_equal(y, (xi @ q.T).astype(np.float64))
    assert np.array_equal(S, (np.abs(xi) @ np.abs(q).T).astype(np.float64))


def test_gemv_q4_matches_exact_rational():
    M, K, N = 2, 64, 3
    x = workloads.activation_bf16(M, K, workload=workloads.Q4_STACK, outliers=0, seed=2)
    w = workloads.master_weights(N, K, workload=workloads.Q4_STACK, seed=2)
    p, s16 = oracle.q4_quant(w)
    y, S = oracle.gemv_q4(x, p, s16)
    q = oracle.q4_unpack(p)
    xv = workloads.bf16_bits_to_f32(x)
    for m in range(M):
        for n in range(N):
            ex = sum(Fraction(float(xv[m, k])) * int(q[n, k]) * Fraction(float(s16[n, k // 32]))
                     for k in range(K))
            assert abs(Fraction(float(y[m, n])) - ex) <= Fraction(2.0 ** -50) * Fraction(float(S[m, n]))
