"""Pins of the FP8 oracle (oracle/fp8.py) against the E4M3 format definition, brute force and closed forms.

E4M3 facts used (OCP 8-bit floating point specification): sign, 4 exponent
bits with bias 7, 3 mantissa bits; largest finite magnitude 448 (0x7E),
smallest normal 2^-6 (0x08), smallest subnormal 2^-9 (0x01), 1.0 = 0x38,
S.1111.111 is NaN.
"""
import math

import numpy as np
import pytest

from oracle import fp8 as F
from expert_routing_grouped_amd import workloads as W


def _brute_encode(v: float) -> int:
    """Nearest finite e4m3 code by scanning all 254 finite codes; ties to the even code."""
    a = min(abs(float(np.float32(v))), 448.0)
    best, best_d = None, None
    for code in range(127):
        e, m = code >> 3, code & 7
        val = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        d = abs(val - a)
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_decode_spec_values():
    dec = F.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0x07, 0x00, 0xFE, 0xB8, 0x39, 0x40], np.uint8))
    assert list(dec) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, 7 / 8 * 2.0 ** -6, 0.0, -448.0, -1.0, 1.125, 2.0]
    assert np.isnan(F.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(F.e4m3_decode(np.array([0x80], np.uint8))[0])
    pos = F.e4m3_positive_values()
    assert len(pos) == 127 and np.all(np.diff(pos) > 0)
    # Between consecutive powers of two above 2^-6 there are exactly 8 values, evenly spaced.
    for e in range(-6, 8):
        seg = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(seg) == 8 and np.allclose(np.diff(seg), 2.0 ** (e - 3))


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = F.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(vals), codes)


def test_encode_matches_brute_force():
    rng = np.random.default_rng(1)
    pos = F.e4m3_positive_values()
    v = np.concatenate([
        rng.standard_normal(400) * 50, rng.standard_normal(400) * 0.02, rng.uniform(-3e-3, 3e-3, 200),
        (pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2,   # every tie
        [448.0, 449.0, 464.0, 1e6, -1e30, 2.0 ** -10, 2.0 ** -10 * 1.0001, -0.0, 0.0],
    ]).astype(np.float32)
    got = F.e4m3_encode(v)
    want = np.array([_brute_encode(x) for x in v], np.uint8)
    assert np.array_equal(got, want)


def test_encode_ties_and_saturation():
    enc = lambda x: int(F.e4m3_encode(np.array([x], np.float32))[0])
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A      # ties to the even code
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02
    assert enc(449.0) == 0x7E and enc(-5000.0) == 0xFE and enc(1e38) == 0x7E


def test_encode_agrees_with_the_generators_quantiser():
    # The input generator rounds with float32 bit arithmetic, the oracle by table
    # search: two independent implementations of the same rounding.
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 1024)) * rng.uniform(0.001, 10, (64, 1))).astype(np.float32)
    x[3, :128] = 0.0
    codes, scales = F.quantize_rows(x)
    gcodes, gscales = W.quantize_e4m3_blocks(x, 1)
    assert np.array_equal(codes, gcodes) and np.array_equal(scales, gscales)


def test_quantize_rows_closed_forms():
    a = np.zeros((3, 256), np.float32)
    a[0, :128] = 0.3                       # constant block: every code 448, scale 0.3 / 448
    a[1, 128:] = -7.0
    codes, scales = F.quantize_rows(a)
    assert (codes[0, :128] == 0x7E).all() and scales[0, 0] == np.float32(np.float32(0.3) / np.float32(448))
    assert (codes[1, 128:] == 0xFE).all() and scales[1, 1] == np.float32(7.0 / 448)
    assert (codes[2] == 0).all() and (scales[2] == 1.0).all()   # all-zero blocks
    assert (codes[0, 128:] == 0).all() and scales[0, 1] == 1.0


def test_quantize_rows_error_bound_and_amax():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((32, 512)) * rng.uniform(0.01, 100, (32, 1))).astype(np.float32)
    codes, scales = F.quantize_rows(a)
    deq = F.dequantize_rows(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    q = a / s
    # Half a unit in the last place of e4m3: |q| / 16 for normals, 2^-10 below 2^-6.
    bound = np.maximum(np.abs(q) / 16, 2.0 ** -10) * s * (1 + 1e-6)
    assert (np.abs(deq - a) <= bound).all()
    blk = np.abs(a).reshape(32, 4, 128)
    arg = blk.argmax(axis=2)
    top = np.take_along_axis(codes.reshape(32, 4, 128), arg[..., None], axis=2)[..., 0]
    assert ((top & 0x7F) == 0x7E).all()    # the largest magnitude of a block maps to 448


def test_dequantize_weights_block_layout():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (256, 384), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    scales = rng.uniform(0.5, 2.0, (2, 3)).astype(np.float32)
    got = F.dequantize_weights(codes, scales)
    for n in (0, 127, 128, 255):
        for k in (0, 129, 255, 256, 383):
            assert got[n, k] == F.e4m3_decode(codes[n:n + 1, k])[0] * float(scales[n // 128, k // 128])


def _decode_scalar(c: int) -> float:
    e, m = (c & 0x7F) >> 3, c & 7
    v = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if c & 0x80 else v


def test_expert_ffn_fp8_brute_force():
    rng = np.random.default_rng(5)
    T, k, d, I, nloc = 4, 2, 256, 128, 2
    x = rng.standard_normal((T, d)).astype(np.float32)
    xq, xs = F.quantize_rows(x)
    wgu = (rng.standard_normal((nloc, 2 * I, d)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((nloc, d, I)) * 0.05).astype(np.float32)
    wgq, wgs = W.quantize_e4m3_blocks(wgu, 128)
    wdq, wds = W.quantize_e4m3_blocks(wd, 128)
    sorted_assign = np.array([1, 4, 7, 0, 5, 2], np.int64)   # assignments t * k + j
    offsets = np.array([0, 3, 6])
    o, hq, hs = F.expert_ffn_fp8(xq, xs, sorted_assign, k, offsets, wgq, wgs, wdq, wds, I)
    for i in range(6):
        t = sorted_assign[i] // k
        e = 0 if i < 3 else 1
        xv = [_decode_scalar(int(xq[t, j])) * float(xs[t, j // 128]) for j in range(d)]
        h = []
        for n in range(I):
            g = sum(xv[j] * _decode_scalar(int(wgq[e, n, j])) * float(wgs[e, n // 128, j // 128]) for j in range(d))
            u = sum(xv[j] * _decode_scalar(int(wgq[e, I + n, j])) * float(wgs[e, (I + n) // 128, j // 128])
                    for j in range(d))
            h.append(np.float32(g / (1 + math.exp(-g)) * u))
        amax = max(abs(v) for v in h)
        sc = np.float32(amax / np.float32(448.0))
        codes = [_brute_encode(np.float32(v / sc)) for v in h]
        assert list(hq[i]) == codes and hs[i, 0] == sc
        hv = [_decode_scalar(c) * float(sc) for c in codes]
        for n in (0, 1, 100, 255):
            want = sum(hv[j] * _decode_scalar(int(wdq[e, n, j])) * float(wds[e, n // 128, j // 128]) for j in range(I))
            assert abs(o[i, n] - want) <= 1e-12 * max(1.0, abs(want))


def test_expert_ffn_fp8_constant_closed_form():
    # All codes 1.0: g = u = d * sx * s1 in every column; h is constant, so its
    # block quantises to 448 exactly; o = I * dequant(h) * s2.
    d, I = 256, 128
    sx, s1, s2 = np.float32(0.01), np.float32(0.002), np.float32(0.003)
    xq = np.full((1, d), 0x38, np.uint8)
    xs = np.full((1, d // 128), sx, np.float32)
    wgq = np.full((1, 2 * I, d), 0x38, np.uint8)
    wgs = np.full((1, 2, 2), s1, np.float32)
    wdq = np.full((1, d, I), 0x38, np.uint8)
    wds = np.full((1, 2, 1), s2, np.float32)
    o, hq, hs = F.expert_ffn_fp8(xq, xs, None, 1, np.array([0, 1]), wgq, wgs, wdq, wds, I)
    g = d * float(sx) * float(s1)
    h32 = np.float32(g / (1 + math.exp(-g)) * g)
    assert (hq == 0x7E).all() and hs[0, 0] == np.float32(h32 / np.float32(448))
    want = I * 448.0 * float(hs[0, 0]) * float(s2)
    assert np.allclose(o, want, rtol=1e-12, atol=0)
