"""Pins for the oracle's block quantisers (live FP8 activation quant, FP8 weight
encode, int4 g32).  Expected values come from the mathematics: the amax element
maps to +-448, each code is the nearest representable value (checked by
exhaustive search over the torch-decoded table), the reconstruction error is at
most half a code step, and the scale is the fp32 quotient amax / 448."""
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
import workloads

E4M3_VALUES = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _nearest_code(r32):
    """Exhaustive nearest-E4M3 search for one fp32 value (ties to even code)."""
    a = Fraction(abs(float(r32)))
    dist = [abs(Fraction(float(x)) - a) for x in E4M3_VALUES]
    m = min(dist)
    best = [c for c, d in enumerate(dist) if d == m]
    c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return c | (0x80 if np.signbit(r32) else 0)


def test_act_quant_shapes_and_scale_rule():
    x = workloads.activation_bf16(3, 512, workload=workloads.FP8_GEMV_SMALL)
    q, s = oracle.act_quant_fp8(x)
    assert q.shape == (3, 512) and q.dtype == np.uint8
    assert s.shape == (3, 4) and s.dtype == np.float32
    xf = workloads.bf16_bits_to_f32(x).reshape(3, 4, 128)
    amax = np.abs(xf).max(axis=2)
    # scale is the correctly rounded fp32 quotient amax/448 (checked in exact rationals)
    for a, sv in zip(amax.ravel(), s.ravel()):
        exact = Fraction(float(a)) / 448
        cand = np.float32(sv)
        up = np.nextafter(cand, np.float32(np.inf))
        dn = np.nextafter(cand, np.float32(0))
        e0 = abs(Fraction(float(cand)) - exact)
        assert e0 <= abs(Fraction(float(up)) - exact) and e0 <= abs(Fraction(float(dn)) - exact)


def test_act_quant_amax_element_hits_448():
    x = workloads.activation_bf16(4, 1024, workload=workloads.FP8_GEMV_SMALL, seed=3)
    q, s = oracle.act_quant_fp8(x)
    xf = workloads.bf16_bits_to_f32(x).reshape(4, 8, 128)
    idx = np.abs(xf).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(4, 8, 128), idx[..., None], axis=2)[..., 0]
    sgn = np.take_along_axis(xf, idx[..., None], axis=2)[..., 0] < 0
    assert np.array_equal(qa, np.where(sgn, 0xFE, 0x7E).astype(np.uint8))


def test_act_quant_codes_are_nearest_and_error_is_half_step():
    x = workloads.activation_bf16(1, 256, workload=workloads.FP8_GEMV_SMALL, seed=5)
    q, s = oracle.act_quant_fp8(x)
    xf = workloads.bf16_bits_to_f32(x)[0]
    for k in range(256):
        r32 = np.float32(xf[k]) / np.float32(s[0, k // 128])
        assert q[0, k] == _nearest_code(r32)
    rec = oracle.dequant_fp8(q, s)[0]
    d = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for k in range(256):
        a = abs(xf[k] / s[0, k // 128])
        i = np.searchsorted(d, a)
        step = d[min(i, 125) + 1] - d[min(i, 125)] if a < 448 else 32.0
        assert abs(rec[k] - xf[k]) <= 0.5 * step * s[0, k // 128] * (1 + 2 ** -20)


def test_act_quant_every_bf16_value_in_a_group():
    """Sweep every finite bf16 pattern as a group member next to a fixed amax."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = workloads.bf16_bits_to_f32(bits)
    finite = np.isfinite(vals) & (np.abs(vals) < 1000.0)
    vals = vals[finite]
    bits = bits[finite]
    n = len(bits) // 127 * 127
    grp = bits[:n].reshape(-1, 127)
    amax_bits = workloads.f32_to_bf16_bits(np.full((grp.shape[0], 1), 1000.0, np.float32))
    x = np.concatenate([grp, amax_bits], axis=1)
    q, s = oracle.act_quant_fp8(x)
    assert np.all(s == np.float32(1000.0) / np.float32(448.0))
    r32 = (workloads.bf16_bits_to_f32(x) / s[:, :1]).astype(np.float32)
    # the oracle's codes equal the torch encoding of the fp32 quotient (|r| <= 448 here)
    ref = torch.from_numpy(r32.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_act_quant_zero_group():
    x = np.zeros((2, 256), np.uint16)
    x[1, 200] = workloads.f32_to_bf16_bits(np.array([3.0], np.float32))[0]
    q, s = oracle.act_quant_fp8(x)
    assert np.all(q[0] == 0) and np.all(s[0] == 1.0)
    assert s[1, 0] == 1.0 and np.all(q[1, :128] == 0)
    assert q[1, 200] == 0x7E and s[1, 1] == np.float32(3.0) / np.float32(448.0)


def test_weight_quant_power_of_two_scaling_is_exact():
    w = workloads.master_weights(8, 256, workload=workloads.FP8_GEMV_SMALL)
    q0, s0 = oracle.block_quant_fp8(w)
    for j in (-3, 5):
        q1, s1 = oracle.block_quant_fp8(w * np.float32(2.0 ** j))
        assert np.array_equal(q0, q1) and np.array_equal(s1, s0 * np.float32(2.0 ** j))


def test_q4_quant_nearest_integer_and_scale_rule():
    w = workloads.master_weights(4, 128, workload=workloads.Q4_STACK)
    p, s16 = oracle.q4_quant(w)
    assert p.shape == (4, 64) and s16.shape == (4, 4) and s16.dtype == np.float16
    q = oracle.q4_unpack(p)
    g = w.reshape(4, 4, 32)
    amax = np.abs(g).max(axis=2)
    assert np.array_equal(s16, (amax / np.float32(7)).astype(np.float16))
    for n in range(4):
        for k in range(128):
            sc = np.float32(s16[n, k // 32])
            r = float(np.float32(w[n, k]) / sc)
            cands = np.arange(-8, 8)
            d = np.abs(cands - r)
            best = cands[d == d.min()]
            expect = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert q[n, k] == expect
    # symmetric quantiser: the amax element maps to +-7
    idx = np.abs(g).argmax(axis=2)
    qa = np.take_along_axis(q.reshape(4, 4, 32), idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(qa) == 7)


def test_q4_zero_group():
    w = np.zeros((1, 64), np.float32)
    w[0, 40] = -0.5
    p, s16 = oracle.q4_quant(w)
    q = oracle.q4_unpack(p)
    assert s16[0, 0] == 0 and np.all(q[0, :32] == 0)
    assert q[0, 40] == -7


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_scale_rounding.txt")


def q4_scale_goldens():
    """(name, amax fp32, expected fp16 bits) from the hand-derived fixture."""
    out = []
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        name, a_hex, s_hex = line.split()[:3]
        amax = np.array([int(a_hex, 16)], np.uint32).view(np.float32)[0]
        out.append((name, amax, int(s_hex, 16)))
    return out


def q4_golden_rows():
    """One 32-value group per golden case: amax at position 5 (negated for odd
    cases), smaller values elsewhere.  Returns (w fp32 [n, 32], expected scale
    bits [n])."""
    cases = q4_scale_goldens()
    w = np.zeros((len(cases), 32), np.float32)
    exp = np.zeros(len(cases), np.uint16)
    for i, (_, amax, sbits) in enumerate(cases):
        row = (np.linspace(-0.9, 0.9, 32) * amax).astype(np.float32)
        row[5] = -amax if i % 2 else amax
        w[i] = row
        exp[i] = sbits
    return w, exp


def test_q4_scale_hand_derived_goldens():
    """The int4 scale rule against hand-derived values at fp16 rounding ties
    (normal, subnormal, overflow): ties to even, no truncation, no rounding
    half away from zero, divisor 7."""
    w, exp = q4_golden_rows()
    p, s16 = oracle.q4_quant(w)
    got = s16[:, 0].view(np.uint16)
    names = [c[0] for c in q4_scale_goldens()]
    for n, g, e in zip(names, got, exp):
        assert g == e, f"case {n}: scale 0x{g:04x}, expected 0x{e:04x}"
    q = oracle.q4_unpack(p)
    for i, e in enumerate(exp):
        if e == 0x7C00:                      # infinite scale: every code 0
            assert np.all(q[i] == 0)
        else:
            # the amax element's code: amax / s rounded to the nearest integer
            # (these quotients are far from .5), clipped; a coarse subnormal
            # scale can put it below 7 (case E: 49/8 -> 6) or above (F: 35/4 -> 7)
            # (the range is asymmetric: -8.75 clips to -8, +8.75 to +7)
            sv = Fraction(float(np.uint16(e).view(np.float16)))
            r = Fraction(float(w[i, 5])) / sv
            assert q[i, 5] == min(max(round(r), -8), 7)


def _fp16_nearest_even(fr):
    """The fp16 nearest to the exact positive rational fr (ties to the even
    mantissa; >= 65520 -> inf), by exact comparison of fr with the fp16
    neighbours of a first guess."""
    if fr >= 65520:
        return 0x7C00
    guess = np.float16(float(fr)).view(np.uint16)
    cands = [int(b) for b in (guess - 1, guess, guess + 1) if 0 <= b < 0x7C00]
    vals = [Fraction(float(np.uint16(b).view(np.float16))) for b in cands]
    d = [abs(v - fr) for v in vals]
    best = [b for b, dd in zip(cands, d) if dd == min(d)]
    return best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]


def test_q4_scale_is_nearest_fp16_to_exact_quotient():
    """For amax spread over fp16's normal and subnormal range, the scale is the
    fp16 nearest to the exact rational amax / 7 (ties to even).  (Rounding the
    fp32 quotient cannot create a tie that the exact quotient does not have:
    neighbouring fp32 quotients of amax / 7 lie at least 4/7 of an fp32 ulp
    apart, so the one fp32 value within half an ulp of an fp16 midpoint is
    the midpoint itself.)"""
    rng = np.random.default_rng(7)
    amax = np.exp2(rng.uniform(-26, 18, size=400)).astype(np.float32)
    w = np.zeros((len(amax), 32), np.float32)
    w[:, 0] = amax
    w[:, 1:] = (rng.uniform(-1, 1, size=(len(amax), 31)) * amax[:, None]).astype(np.float32)
    _, s16 = oracle.q4_quant(w)
    for a, s in zip(amax, s16[:, 0].view(np.uint16)):
        assert s == _fp16_nearest_even(Fraction(float(a)) / 7), f"amax {a!r}: scale 0x{s:04x}"
