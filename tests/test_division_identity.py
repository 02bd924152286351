"""The FP8 quantisers divide by a block scale s as RN32(RN64(v * RN64(1 / s))): one float64
reciprocal per block and a float64 multiply per value, in place of the float32 division the
quantisation rule is stated with. For float32 v and s the two are equal (the float64 product is
within 2^-51.9 of v / s, and a quotient of two float32 values that is not itself a float32 lies
at least 2^-49 away from every float32 rounding midpoint, relative). This checks the identity
on the CPU: random operands over the quantiser's ranges (s = RN32(amax / 448), |v| <= amax,
30 decades), operands whose quotient sits on or next to an e4m3 rounding midpoint, and every
significand of v in [1, 2) against a set of scales.
"""
import numpy as np


def _same(v, s):
    v = np.asarray(v, np.float32)
    s = np.asarray(s, np.float32)
    ref = v / s
    got = (v.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)
    return np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_random_scales_and_values():
    rng = np.random.default_rng(11)
    for _ in range(8):
        amax = np.abs(rng.standard_normal(1 << 20).astype(np.float32)
                      * (np.float32(10.0) ** rng.uniform(-30, 30, 1 << 20).astype(np.float32)))
        amax += np.float32(1e-30)
        s = (amax / np.float32(448.0)).astype(np.float32)
        v = (amax * rng.uniform(-1, 1, amax.size).astype(np.float32)).astype(np.float32)
        assert _same(v, s)


def test_quotients_at_e4m3_midpoints():
    rng = np.random.default_rng(12)
    # e4m3 rounding midpoints (between consecutive codes) and the codes themselves
    pos = np.array([(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)] +
                   [m / 8 * 2.0 ** -6 for m in range(1, 8)], np.float64)
    pos = np.sort(pos[pos <= 448])
    targets = np.concatenate([pos, (pos[1:] + pos[:-1]) / 2])
    s = (np.abs(rng.standard_normal(1 << 16)) * 10.0 ** rng.uniform(-8, 8, 1 << 16)).astype(np.float32)
    for t in targets:
        v = (s * np.float32(t)).astype(np.float32)
        assert _same(v, s)
        assert _same(np.nextafter(v, np.float32(np.inf)), s)
        assert _same(np.nextafter(v, np.float32(-np.inf)), s)


def test_every_significand():
    rng = np.random.default_rng(13)
    sig = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(127 << 23)).view(np.float32)   # [1, 2)
    for sv in rng.uniform(1, 2, 4).astype(np.float32):
        assert _same(sig, np.full(sig.size, sv, np.float32))
