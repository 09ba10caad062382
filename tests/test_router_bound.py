"""The certified router's error bound, checked in exact arithmetic on the CPU.

From 256 tokens the HIP router takes logits from int8 slices of x and W_r and
keeps a top-k only when every gap among the best k + 1 keys exceeds twice a
per-token bound (else the token is recomputed exactly).  Routing is exact only
if that bound really covers |our logit - the oracle's logit|.  These tests
restate the slicing from its definition (each row scaled by 2^-a, a its
exponent, then cut by truncation into NSL = 5 signed 7-bit slices; the
slice pairs with p + q <= 4 are kept), evaluate it in rational arithmetic and in the
fp64 order the kernels use, and check against both the exact dot product and
the oracle's sequential fp64 sum:

    |ours - exact|  <= 2^a_x 2^-35 (5 d 2^a_w + |w|_1)                 (slicing)
    |ours - oracle| <= that + (2 d + 128 + 32 S) 2^-53 2^a_x |w|_1     (fp64 sums)

on random rows, rows at the top of their binade (largest truncation), rows
with one large and many tiny entries, same-sign rows whose dropped slice
pairs and truncated bits all add up (they reach ~10 % of the bound, so a
bound ten times too small fails), and several K splits S.  Test code only:
it shares nothing with the HIP sources."""
from fractions import Fraction

import numpy as np
import pytest

NSL = 5  # slices per operand


def _exponent(row):
    m = float(np.max(np.abs(row)))
    if m == 0.0:
        return None
    _, e = np.frexp(np.float32(m))  # m = f 2^e, 0.5 <= f < 1: m < 2^e
    return int(e)


def _slices(row):
    """int slices V[p][i] with row = 2^a (sum_p V_p 2^-7(p+1) + r 2^-7NSL)."""
    a = _exponent(row)
    if a is None:
        return None, np.zeros((NSL, row.size), dtype=np.int64)
    u = np.ldexp(row.astype(np.float32), -a).astype(np.float32)  # exact
    out = np.zeros((NSL, row.size), dtype=np.int64)
    for p in range(NSL):
        t = (u * np.float32(128.0)).astype(np.float32)  # exact
        q = np.trunc(t).astype(np.float32)
        out[p] = q.astype(np.int64)
        u = (t - q).astype(np.float32)                   # exact: the fraction
    return a, out


def _ours_fp64(x, w, nsplit):
    """The kernels' evaluation order: per K slice, NSL int32 level sums
    (p + q = l), added in fp64 from l = NSL - 1 down, scaled by 2^(a_x + a_w); the
    slices' results added in slice order."""
    ax, X = _slices(x)
    aw, W = _slices(w)
    if ax is None or aw is None:
        return 0.0
    d = x.size
    kc = d // nsplit
    total = 0.0
    for s in range(nsplit):
        ks = slice(s * kc, (s + 1) * kc)
        acc = [0] * NSL
        for p in range(NSL):
            for q in range(NSL - p):
                acc[p + q] += int(np.dot(X[p, ks], W[q, ks]))
        part = 0.0
        for lev in range(NSL - 1, -1, -1):
            assert abs(acc[lev]) < 2**31  # the int32 accumulators cannot overflow
            part += np.ldexp(float(acc[lev]), -7 * (lev + 2))
        part = np.ldexp(part, ax + aw)
        total = part if s == 0 else total + part
    return total


def _ours_exact(x, w):
    """The same kept slice pairs in rational arithmetic (no fp64 rounding)."""
    ax, X = _slices(x)
    aw, W = _slices(w)
    if ax is None or aw is None:
        return Fraction(0)
    v = Fraction(0)
    for p in range(NSL):
        for q in range(NSL - p):
            v += Fraction(int(np.dot(X[p], W[q])), 2 ** (7 * (p + q + 2)))
    return v * Fraction(2) ** (ax + aw)


def _exact(x, w):
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w)), Fraction(0))


def _oracle_fp64(x, w):
    acc = 0.0
    for a, b in zip(x, w):
        acc += float(a) * float(b)  # fp32 x fp32 is exact in fp64
    return acc


def _bounds(x, w, nsplit):
    ax, aw = _exponent(x), _exponent(w)
    if ax is None or aw is None:
        return 0.0, 0.0
    d = x.size
    w1 = float(np.sum(np.abs(w.astype(np.float64))))
    trunc = 2.0 ** ax * 2.0 ** (-7 * NSL) * (NSL * d * 2.0 ** aw + w1)
    rnd = (2 * d + 128 + 32 * nsplit) * 2.0 ** -53 * 2.0 ** ax * w1
    return trunc, rnd


def _rows(kind, d, rng):
    if kind == "normal":
        return rng.standard_normal(d).astype(np.float32), (rng.standard_normal(d) / np.sqrt(d)).astype(np.float32)
    if kind == "top_of_binade":
        # every entry just below a power of two: the most bits past the slices
        x = (np.float32(np.nextafter(np.float32(2.0), np.float32(0))) *
             rng.choice([-1.0, 1.0], d)).astype(np.float32)
        w = (np.float32(np.nextafter(np.float32(0.125), np.float32(0))) *
             rng.choice([-1.0, 1.0], d)).astype(np.float32)
        return x, w
    if kind == "spiky":
        # one large entry sets the exponent; the rest fall below the slices
        x = (rng.standard_normal(d) * 1e-9).astype(np.float32)
        x[0] = np.float32(3.75)
        w = (rng.standard_normal(d) * 1e-7).astype(np.float32)
        w[d // 2] = np.float32(-1.5)
        return x, w
    if kind == "aligned_top":
        # same sign everywhere, every mantissa all ones: the dropped slice
        # pairs (p + q >= NSL) all add up instead of cancelling
        x = np.full(d, np.nextafter(np.float32(2.0), np.float32(0)), np.float32)
        w = np.full(d, np.nextafter(np.float32(0.125), np.float32(0)), np.float32)
        return x, w
    if kind == "aligned_spiky":
        # one large entry sets the exponent; the small positive rest carry
        # bits below the kept slices, all truncated the same way
        x = np.full(d, np.float32(1.2345678e-10) * np.float32(7.0), np.float32)
        x[0] = np.float32(3.75)
        w = rng.uniform(0.5, 1.0, d).astype(np.float32)
        return x, w
    if kind == "ragged_mantissas":
        x = rng.uniform(-1, 1, d).astype(np.float32) * np.float32(2.0 ** 20)
        w = rng.uniform(-1, 1, d).astype(np.float32) * np.float32(2.0 ** -30)
        return x, w
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "top_of_binade", "spiky", "ragged_mantissas", "aligned_top",
                                  "aligned_spiky"])
@pytest.mark.parametrize("d,nsplit", [(64, 1), (256, 1), (256, 4), (512, 8)])
def test_sliced_logit_within_the_certified_bound(kind, d, nsplit):
    rng = np.random.default_rng([d, nsplit, len(kind)])
    for _ in range(4):
        x, w = _rows(kind, d, rng)
        trunc, rnd = _bounds(x, w, nsplit)
        exact = _exact(x, w)
        # slicing alone, in exact arithmetic
        assert abs(_ours_exact(x, w) - exact) <= Fraction(trunc)
        # the kernels' fp64 evaluation against the oracle's fp64 sum
        ours = _ours_fp64(x, w, nsplit)
        assert abs(ours - _oracle_fp64(x, w)) <= trunc + rnd


def test_zero_rows_give_zero():
    d = 128
    z = np.zeros(d, np.float32)
    v = np.ones(d, np.float32)
    assert _ours_fp64(z, v, 2) == 0.0 and _ours_fp64(v, z, 1) == 0.0
    assert _bounds(z, v, 1) == (0.0, 0.0)


def test_truncated_slices_never_exceed_the_value():
    """The fp64 part of the bound takes every kept slice product no larger in
    magnitude than the value it slices (truncation toward zero)."""
    rng = np.random.default_rng(7)
    row = (rng.standard_normal(1000) * 3).astype(np.float32)
    a, S = _slices(row)
    for p in range(NSL):
        sl = S[p].astype(np.float64) * 2.0 ** (a - 7 * (p + 1))
        rem = row.astype(np.float64) - sum(S[q].astype(np.float64) * 2.0 ** (a - 7 * (q + 1)) for q in range(p))
        assert np.all(np.abs(sl) <= np.abs(rem) + 0.0)
        assert np.all(np.abs(sl) <= np.abs(row.astype(np.float64)) + 0.0)
