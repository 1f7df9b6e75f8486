"""Weight-streaming linear layers: block-scaled FP8 GEMV, int4 g32 GEMV, SiLU(gate)*up.

Test infrastructure (see the package docstring).

Each linear is computed the plainest way: dequantise both operands to float64
(exact, see below) and take one float64 matrix product.  This is the result
the method reaches up to rounding order: [Sionic] (intro and §2) streams every
weight once and applies one scale per K block; multiplying the scale into
every element first is the same sum regrouped.

Precision: a dequantised FP8 value has at most 4 + 24 significant bits, so it
is exact in float64; the product of two has at most 56 bits and is rounded
once, and the float64 sum over K adds at most K * 2^-53 * S of error, where S
is the error scale returned alongside (S[m, n] = sum_k |x~[m,k]| * |w~[n,k]|).
For K <= 32768 that is below 4e-12 * S, far inside any tolerance used here.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_to_f64
from .quant import dequant_fp8, dequant_q4


def gemv_fp8(qx, sx, qw, sw):
    """y[m, n] = sum_k (qx[m,k]*sx[m,k/128]) * (qw[n,k]*sw[n,k/128]).

    qx uint8 [M, K], sx fp32 [M, K/128], qw uint8 [N, K] (row-major weight rows),
    sw fp32 [N, K/128].  Returns (y float64 [M, N], S float64 [M, N]).
    """
    xt = dequant_fp8(np.atleast_2d(qx), np.atleast_2d(sx))
    wt = dequant_fp8(qw, sw)
    return xt @ wt.T, np.abs(xt) @ np.abs(wt).T


def silu_mul(y, inter: int | None = None):
    """h = silu(gate) * up for a gate||up row block ([Sionic] §1 names the fused
    expert gate_up GEMM; the epilogue itself is not detailed on the pages).

    Reading taken: rows [0, I) of the gate_up output are the gate, rows [I, 2I)
    the up projection; silu(g) = g * sigmoid(g) = g / (1 + exp(-g)); float64.
    """
    y = np.asarray(y, dtype=np.float64)
    I = y.shape[-1] // 2 if inter is None else inter
    g = y[..., :I]
    u = y[..., I:2 * I]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def gemv_q4(x_bf16_bits, packed, scales16):
    """W4A16 GEMV: y[m, n] = sum_k x[m,k] * q[n,k] * s[n,k/32], x bf16 [M, K].

    Returns (y float64 [M, N], S float64 [M, N]); every product is exact in
    float64 (8 + 4 + 11 significant bits).
    """
    x = bf16_bits_to_f64(np.atleast_2d(x_bf16_bits))
    wt = dequant_q4(packed, scales16)
    return x @ wt.T, np.abs(x) @ np.abs(wt).T
