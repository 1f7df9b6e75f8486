"""CPU model of the wave reductions the GPU kernels use for their sums (test
infrastructure: the model restates the lane exchanges, not the kernels'
code).

A wave is 64 lanes of float32.  The transposing butterfly takes N values per
lane (N a power of two): at the stage of lane distance d = 2^s a lane keeps
the half of its values whose index bit s equals its lane bit s and adds its
partner's (lane l ^ d) copy of them; once one value is left the remaining
distances add it as a plain butterfly.  The claims checked here are what the
kernels' bitwise guarantees rest on:

* lane l ends with the sum of value l mod N;
* every value's sum has the same bits whatever N and whatever its index (so
  a token's sums do not depend on how many tokens share the reduction);
* a segment sum over an aligned group of 2^k lanes, with the 8- and 16-lane
  stages taking their partner from the row mirrors, equals the full-wave sum
  of that row placed alone in the wave (other lanes zero);
* the row rotations by 4 and 12 give lane l ^ 4 where the kernels take them.
"""
import numpy as np

LANES = 64


def xor_partner(v, d):
    """v[l ^ d] for every lane l (float32 array of 64)."""
    idx = np.arange(LANES) ^ d
    return v[idx]


def butterfly_many(vals):
    """vals: float32 [N, 64] (value i held by every lane).  Returns the
    float32 [64] each lane ends with."""
    n = vals.shape[0]
    lane = np.arange(LANES)
    c = [vals[i].astype(np.float32).copy() for i in range(n)]
    for s in range(6):
        d = 1 << s
        if len(c) > 1:
            hi = ((lane >> s) & 1).astype(bool)
            nc = []
            for i in range(len(c) // 2):
                keep = np.where(hi, c[2 * i + 1], c[2 * i])
                send = np.where(hi, c[2 * i], c[2 * i + 1])
                nc.append((keep + xor_partner(send, d)).astype(np.float32))
            c = nc
        else:
            c[0] = (c[0] + xor_partner(c[0], d)).astype(np.float32)
    return c[0]


def row_mirror(v, width):
    """Lane l reads lane (width - 1 - l mod width) of its aligned group."""
    lane = np.arange(LANES)
    base = lane - lane % width
    return v[base + (width - 1 - lane % width)]


def segment_sum(v, lanes):
    v = v.astype(np.float32).copy()
    v = (v + xor_partner(v, 1)).astype(np.float32)
    if lanes >= 4:
        v = (v + xor_partner(v, 2)).astype(np.float32)
    if lanes >= 8:
        v = (v + row_mirror(v, 8)).astype(np.float32)
    if lanes >= 16:
        v = (v + row_mirror(v, 16)).astype(np.float32)
    if lanes >= 32:
        v = (v + xor_partner(v, 16)).astype(np.float32)
    if lanes >= 64:
        v = (v + xor_partner(v, 32)).astype(np.float32)
    return v


def _rand(rng, shape):
    # wide magnitudes and both signs, so that the order of additions shows in the bits
    return (rng.standard_normal(shape) * 2.0 ** rng.integers(-20, 20, size=shape)).astype(np.float32)


def test_lane_holds_its_value_sum():
    rng = np.random.default_rng(1)
    for n in (1, 2, 4, 8, 16):
        vals = _rand(rng, (n, LANES))
        out = butterfly_many(vals)
        for lane in range(LANES):
            want = np.sum(vals[lane % n].astype(np.float64))
            assert abs(float(out[lane]) - want) <= 1e-5 * np.sum(np.abs(vals[lane % n].astype(np.float64)))


def test_value_bits_do_not_depend_on_width_or_index():
    rng = np.random.default_rng(2)
    for trial in range(20):
        row = _rand(rng, (LANES,))
        ref = None
        for n in (1, 2, 4, 8, 16):
            for pos in range(n):
                vals = _rand(rng, (n, LANES))
                vals[pos] = row
                got = butterfly_many(vals)[pos]      # lane pos holds value pos
                if ref is None:
                    ref = got
                assert got.view(np.uint32) == ref.view(np.uint32), (trial, n, pos)


def test_segment_sum_equals_the_row_alone_in_the_wave():
    rng = np.random.default_rng(3)
    for lanes in (8, 16, 32):
        for trial in range(20):
            v = _rand(rng, (LANES,))
            seg = segment_sum(v, lanes)
            for g in range(LANES // lanes):
                alone = np.zeros(LANES, np.float32)
                alone[g * lanes:(g + 1) * lanes] = v[g * lanes:(g + 1) * lanes]
                full = butterfly_many(alone[None, :])
                part = seg[g * lanes:(g + 1) * lanes]
                assert np.all(part.view(np.uint32) == full[g * lanes].view(np.uint32)), (lanes, trial, g)


def test_row_rotations_give_the_distance_4_partner():
    # a row rotation by r: lane l reads lane (l - r) mod 16 of its row (the
    # layout an in-bounds probe measured on the device)
    lane = np.arange(LANES)
    row = lane - lane % 16
    ror4 = row + (lane - 4) % 16
    ror12 = row + (lane - 12) % 16
    partner = np.where(lane & 4, ror4, ror12)
    assert np.array_equal(partner, lane ^ 4)
    ror8 = row + (lane - 8) % 16
    assert np.array_equal(ror8, lane ^ 8)
