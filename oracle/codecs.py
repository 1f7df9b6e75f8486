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


def _e4m3_value(c: int) -> float:
    """Value of one E4M3FN byte from the format definition (NaN for 0x7F/0xFF).

    Byte layout s|eeee|mmm.  Exponent field 0 is subnormal: (-1)^s * 2^-6 * m/8.
    Exponent fields 1..15 are normal: (-1)^s * 2^(e-7) * (1 + m/8), except that
    e=15, m=7 is NaN.  There is no infinity.  (OCP OFP8 definition of E4M3.)
    """
    s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 0x7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


# the 256 decoded values, and the 126 midpoints between consecutive non-negative finite values
_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
_E4M3_MIDPOINTS = (_E4M3_TABLE[1:0x7F] + _E4M3_TABLE[0:0x7E]) / 2.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3FN byte, as float64 (NaN for 0x7F and 0xFF)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(values) -> np.ndarray:
    """Encode float32 values to E4M3FN bytes.

    Rounding is to the nearest representable magnitude with ties to the even
    code (the even mantissa), found by bisection over the midpoints between
    consecutive codes; magnitudes beyond the largest midpoint (including all
    values at or above 448, and infinities) take the largest finite code 0x7E
    ("satfinite"); NaN encodes to 0x7F; the sign bit is copied.  The pages give
    no rounding or overflow rule; this is the reading taken (round to nearest
    even is the IEEE default, saturation keeps a scaled block finite).
    """
    v = np.asarray(values, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    c = np.searchsorted(_E4M3_MIDPOINTS, a, side="left")       # mids[c-1] < a <= mids[c]
    mid = _E4M3_MIDPOINTS[np.minimum(c, len(_E4M3_MIDPOINTS) - 1)]
    tie = (c < len(_E4M3_MIDPOINTS)) & (a == mid)
    c = np.where(tie & (c % 2 == 1), c + 1, c)                  # a tie goes to the even code
    code = c.astype(np.uint8) | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


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
