"""Exact number codecs used by the decode path: FP8 E4M3, bf16, int4 nibbles.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the CPU baseline of the bench.

The pages only say "FP8" for the live activation quantisation ([Sionic] §1 and
§8c) and for the LM head ([Sionic] §8b).  Reading taken: the OCP 8-bit floating
point format E4M3 in its "FN" flavour (finite only, max 448, one NaN pattern
per sign), which is what MI355X (gfx950) converts natively.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_NORMAL = 2.0 ** -6
_E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3FN byte, as float64 (NaN for 0x7F and 0xFF).

    Byte layout s|eeee|mmm.  Exponent field 0 is subnormal: (-1)^s * 2^-6 * m/8.
    Exponent fields 1..15 are normal: (-1)^s * 2^(e-7) * (1 + m/8), except that
    e=15, m=7 is NaN.  There is no infinity.  (OCP OFP8 definition of E4M3.)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e4m3_encode(values) -> np.ndarray:
    """Encode float32 values to E4M3FN bytes.

    Rounding is to nearest with ties to even on the 3-bit mantissa (the
    subnormal grid is 2^-9); magnitudes at or above 448 saturate to 448
    ("satfinite"); NaN encodes to 0x7F.  The pages give no rounding or overflow
    rule; this is the reading taken (round-to-nearest-even is the IEEE default,
    saturation keeps a scaled block finite).
    """
    v = np.asarray(values, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)

    # subnormal range: count multiples of 2^-9, round half to even
    n_sub = np.rint(a / _E4M3_SUBNORMAL_QUANTUM)            # 0..8; 8 is the first normal
    # normal range: a = 2^e * (1 + f), round f to 3 bits
    safe = np.where((a > 0) & np.isfinite(a), a, 1.0)
    frac, ex = np.frexp(safe)                  # safe = frac * 2^ex, 0.5 <= frac < 1 (exact)
    e = ex.astype(np.int64) - 1                # safe = (2*frac) * 2^e, 1 <= 2*frac < 2
    mant = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)   # 0..8, exact scaling
    e = np.where(mant == 8, e + 1, e)
    mant = np.where(mant == 8, 0, mant)
    code_norm = ((e + 7) << 3) | mant

    n_sub = np.where(a < _E4M3_MIN_NORMAL, n_sub, 0.0).astype(np.int64)
    code = np.where(a < _E4M3_MIN_NORMAL, n_sub, code_norm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.minimum(code, 0x7E)
    code = code | sign
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def bf16_round(values) -> np.ndarray:
    """Round float64 (or float32) values to the nearest bf16, ties to even, in one step.

    bf16 has 8 significant bits and the float32 exponent range (subnormal
    quantum 2^-133).  Results are returned as float64 holding the bf16 value.
    Overflow past the largest finite bf16 gives +-inf.
    """
    v = np.asarray(values, dtype=np.float64)
    finite = np.isfinite(v) & (v != 0)
    safe = np.where(finite, v, 1.0)
    _, e = np.frexp(safe)                      # safe = f * 2^e, 0.5 <= |f| < 1
    q = np.maximum(e - 8, -133)                # exponent of one bf16 ulp
    r = np.ldexp(np.rint(np.ldexp(safe, -q)), q)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    return np.where(finite, r, v)


def bf16_bits(values) -> np.ndarray:
    """bf16 bit patterns (uint16) of ``bf16_round(values)``."""
    r = bf16_round(values).astype(np.float32)   # exact: r is representable in bf16
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns as float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def q4_pack(q) -> np.ndarray:
    """Pack signed int4 values q in [-8, 7] along the last axis into bytes.

    Reading taken (the pages only name Q4 / K4 / AWQ INT4 formats): offset
    binary nibbles u = q + 8; the low nibble of byte j holds element 2j and the
    high nibble element 2j+1.
    """
    q = np.asarray(q, dtype=np.int64)
    assert q.shape[-1] % 2 == 0
    assert q.min(initial=0) >= -8 and q.max(initial=0) <= 7
    u = (q + 8).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def q4_unpack(packed) -> np.ndarray:
    """Inverse of :func:`q4_pack`: bytes [..., K/2] -> int64 [..., K] in [-8, 7]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo = (p & 0xF) - 8
    hi = (p >> 4) - 8
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out
