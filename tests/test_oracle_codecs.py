"""Pins for the oracle codecs (FP8 E4M3FN, bf16, int4 nibbles).

The expected values never come from the oracle itself: they come from torch's
float8_e4m3fn / bfloat16 conversions (an independent library), from a brute
force nearest-value search over the decoded code table, or from exact rational
arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_e4m3_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_torch():
    ours = oracle.e4m3_decode(ALL_CODES)
    ref = torch_e4m3_decode(ALL_CODES)
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_o, nan_r)
    assert np.array_equal(ours[~nan_o], ref[~nan_r])
    # signed zero
    assert np.array_equal(np.signbit(ours[~nan_o]), np.signbit(ref[~nan_r]))


def test_e4m3_table_landmarks():
    d = oracle.e4m3_decode(ALL_CODES)
    assert np.isnan(d).sum() == 2 and np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isfinite(d).sum() == 254
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert d[0x38] == 1.0


def _brute_force_encode(values32):
    """Nearest finite E4M3 value by exhaustive search, ties to the even code."""
    # exact integer arithmetic: every fp32 and every E4M3 value is a multiple of 2^-149
    d = [int(Fraction(float(x)) * 2 ** 149) for x in torch_e4m3_decode(ALL_CODES[:0x7F])]
    out = np.empty(len(values32), dtype=np.uint8)
    for i, v in enumerate(np.asarray(values32, dtype=np.float32)):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        if np.isinf(v):
            c = 0x7E
        else:
            a = int(Fraction(abs(float(v))) * 2 ** 149)
            dist = [abs(x - a) for x in d]
            dmin = min(dist)
            best = [c for c, x in enumerate(dist) if x == dmin]
            c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | (0x80 if np.signbit(v) else 0)
    return out


def _probe_values():
    d = oracle.e4m3_decode(ALL_CODES[:0x7F])
    mids = ((d[1:] + d[:-1]) / 2).astype(np.float32)  # exact in fp32 (<= 5 significant bits)
    assert np.array_equal(mids.astype(np.float64), (d[1:] + d[:-1]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    grid = d.astype(np.float32)
    rng = np.random.default_rng(1234)
    rnd = np.exp2(rng.uniform(-14, 10, 4000)).astype(np.float32)
    big = np.array([448.0, 449.0, 463.99, 464.0, 465.0, 1e6, 3.0e38, np.inf], np.float32)
    tiny = np.array([0.0, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 2.0 ** -11, 1e-30, 1e-45], np.float32)
    v = np.concatenate([mids, up, dn, grid, rnd, big, tiny])
    return np.concatenate([v, -v, np.array([np.nan], np.float32)])


def test_e4m3_encode_matches_brute_force_nearest():
    v = _probe_values()
    assert np.array_equal(oracle.e4m3_encode(v), _brute_force_encode(v))


def test_e4m3_encode_matches_torch_in_range():
    v = _probe_values()
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


def test_e4m3_roundtrip_every_code():
    finite = ALL_CODES[np.isfinite(oracle.e4m3_decode(ALL_CODES))]
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(finite).astype(np.float32)), finite)


def test_bf16_round_matches_torch_for_fp32_inputs():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
                        np.exp2(rng.uniform(-140, 127, 5000)).astype(np.float32),
                        np.array([0.0, -0.0, 3.3895e38, 3.4e38, 1e-40], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), ref)
    ref_bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits(v.astype(np.float64)), ref_bits)


def _bf16_neighbours(bits):
    b = int(bits)
    def val(x):
        return float(np.array([x << 16], np.uint32).view(np.float32)[0])
    return val(b), val(b - 1) if (b & 0x7FFF) else -val(b), val(b + 1)


def test_bf16_round_is_nearest_even_for_fp64_inputs():
    """Exact rational check, including doubles that an fp32 intermediate would
    round onto a bf16 midpoint (double-rounding traps)."""
    rng = np.random.default_rng(9)
    base = rng.standard_normal(300)
    mids = []
    for b in rng.integers(0x3F00, 0x4100, 100):
        lo = float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(int(b) + 1) << 16], np.uint32).view(np.float32)[0])
        m = (lo + hi) / 2
        mids += [m, m * (1 + 2.0 ** -40), m * (1 - 2.0 ** -40)]
    vals = np.concatenate([base, np.array(mids)])
    r = oracle.bf16_round(vals)
    bits = oracle.bf16_bits(vals)
    for v, rv, bv in zip(vals, r, bits):
        here, below, above = _bf16_neighbours(bv)
        assert rv == here
        fv = Fraction(float(v))
        d0 = abs(fv - Fraction(here))
        assert d0 <= abs(fv - Fraction(below)) and d0 <= abs(fv - Fraction(above))
        if d0 in (abs(fv - Fraction(below)), abs(fv - Fraction(above))) and d0 != 0:
            assert int(bv) % 2 == 0            # tie -> even


def test_q4_pack_unpack_all_bytes():
    q = oracle.q4_unpack(ALL_CODES[None, :])[0]
    assert q.min() == -8 and q.max() == 7
    # low nibble is the even element
    assert np.array_equal(q[0::2], (ALL_CODES & 0xF).astype(np.int64) - 8)
    assert np.array_equal(q[1::2], (ALL_CODES >> 4).astype(np.int64) - 8)
    assert np.array_equal(oracle.q4_pack(q[None, :])[0], ALL_CODES)


def test_q4_all_sixteen_codes_decode():
    vals = np.arange(-8, 8)
    packed = oracle.q4_pack(np.repeat(vals, 2)[None, :])
    assert np.array_equal(oracle.q4_unpack(packed)[0], np.repeat(vals, 2))


@pytest.mark.parametrize("bad", [-9, 8])
def test_q4_pack_rejects_out_of_range(bad):
    with pytest.raises(AssertionError):
        oracle.q4_pack(np.array([[bad, 0]]))
