"""Pins of the oracle's MXFP4 quantiser (OCP MX conversion: shared exponent
floor(log2 amax) - 2, round-to-nearest-even onto the E2M1 grid, saturation
at 6): constructed ties, grid round trips, amax edges, zero blocks, and a
brute-force nearest-value search."""
import numpy as np
import pytest

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _brute_code(m: float, neg: bool) -> int:
    """Nearest grid value by exhaustive distance; exact ties pick the even index."""
    dist = np.abs(GRID - min(m, 6.0))
    best = np.flatnonzero(dist == dist.min())
    idx = int(best[0]) if len(best) == 1 else int([i for i in best if i % 2 == 0][0])
    return (8 if neg else 0) | idx


def _brute_block(v):
    v = np.asarray(v, np.float64)
    amax = np.abs(v).max()
    if amax == 0:
        return [8 if np.signbit(a) else 0 for a in v], 0
    # floor(log2 amax) by exact power-of-two comparisons (np.log2 rounds up
    # just below a power of two)
    p = 0
    while 2.0 ** (p + 1) <= amax:
        p += 1
    while 2.0 ** p > amax:
        p -= 1
    e = p - 2
    byte = min(max(e + 127, 0), 254)
    return [_brute_code(abs(a) / 2.0 ** (byte - 127), np.signbit(a)) for a in v], byte


def _codes_list(c):
    c = c.reshape(-1)
    out = []
    for b in c:
        out += [int(b) & 15, int(b) >> 4]
    return out


def _check(v):
    c, s = oracle.mx_quantize(np.asarray(v).reshape(1, -1))
    bc, bs = _brute_block(v)
    assert int(s[0, 0]) == bs
    assert _codes_list(c) == bc


def test_every_midpoint_rounds_to_even():
    # amax = 4 fixes scale byte 127; then put every midpoint in the block
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect_idx = [0, 2, 2, 4, 4, 6, 6]
    v = np.zeros(32)
    v[0] = 4.0
    v[1:8] = mids
    v[8:15] = [-m for m in mids]
    c, s = oracle.mx_quantize(v.reshape(1, -1))
    assert s[0, 0] == 127
    got = _codes_list(c)
    assert got[1:8] == expect_idx
    assert got[8:15] == [8 | i for i in expect_idx]
    _check(v)


def test_grid_values_round_trip_exactly():
    for byte in (1, 100, 127, 140, 254):
        v = np.zeros(32)
        sc = 2.0 ** (byte - 127)
        v[:8] = GRID * sc
        v[8:16] = -GRID * sc
        v[16] = 6.0 * sc  # keep amax at 6 * scale
        c, s = oracle.mx_quantize(v.reshape(1, -1))
        assert s[0, 0] == byte
        back = oracle.mx_dequant(c.reshape(1, -1), s.reshape(1, -1))[0]
        assert np.array_equal(back, v)


@pytest.mark.parametrize("k", [-20, -1, 0, 3, 30])
def test_amax_edges(k):
    for amax, top_idx in ((4 * 2.0 ** k, 6), (6 * 2.0 ** k, 7), (np.nextafter(8.0, 0) * 2.0 ** k, 7)):
        v = np.zeros(32)
        v[5] = amax
        v[6] = -amax
        c, s = oracle.mx_quantize(v.reshape(1, -1))
        assert s[0, 0] == k + 127
        codes = _codes_list(c)
        assert codes[5] == top_idx and codes[6] == 8 | top_idx
        _check(v)


def test_zero_and_negative_zero_blocks():
    c, s = oracle.mx_quantize(np.zeros((1, 32)))
    assert s[0, 0] == 0 and np.all(c == 0)
    c, s = oracle.mx_quantize(np.full((1, 32), -0.0))
    assert s[0, 0] == 0 and np.all(c == 0x88)
    # negative values that round to zero keep the sign bit
    v = np.zeros(32)
    v[0] = 4.0
    v[1] = -0.1
    assert _codes_list(oracle.mx_quantize(v.reshape(1, -1))[0])[1] == 8


def test_scale_byte_clamps():
    v = np.zeros(32)
    v[0] = 2.0 ** 200            # fp64 only: e + 127 > 254 -> clamp to 254, saturate
    c, s = oracle.mx_quantize(v.reshape(1, -1))
    assert s[0, 0] == 254 and _codes_list(c)[0] == 7
    v[0] = 2.0 ** -140           # e + 127 < 0 -> clamp to 0
    c, s = oracle.mx_quantize(v.reshape(1, -1))
    assert s[0, 0] == 0
    _check(v)


def test_fp32_subnormal_block():
    v = np.zeros(32, np.float32)
    v[3] = np.float32(1e-40)      # fp32 subnormal: widened exactly
    v[4] = np.float32(-3e-41)
    _check(v.astype(np.float64))


def test_random_blocks_vs_brute_force():
    r = np.random.default_rng(21)
    for scale in (1e-3, 1.0, 1e3):
        v = (r.standard_normal((64, 32)) * scale).astype(np.float32).astype(np.float64)
        c, s = oracle.mx_quantize(v)
        for b in range(64):
            bc, bs = _brute_block(v[b])
            assert int(s[b, 0]) == bs and _codes_list(c[b]) == bc


def test_roundtrip_error_bound():
    r = np.random.default_rng(22)
    v = r.standard_normal((200, 32)).astype(np.float32).astype(np.float64)
    c, s = oracle.mx_quantize(v)
    back = oracle.mx_dequant(c, s)
    sc = 2.0 ** (s.astype(np.float64) - 127)
    # every magnitude below 6*scale lands within half a grid step (step <= 2*scale)
    err = np.abs(back - v)
    within = np.abs(v) <= 6 * np.repeat(sc, 32, axis=1)
    assert np.all(err[within] <= np.repeat(sc, 32, axis=1)[within] * 1.0 + 0)
