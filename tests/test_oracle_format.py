"""Pins of the oracle's MXFP4 decode (E2M1 codes, E8M0 scales, packing)
against what the pages print and what the OCP MX bit layout fixes."""
import os
import struct

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_numbers(name):
    vals = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(line)
    return vals


def _ocp_e2m1_from_bits(code: int) -> float:
    """E2M1 from its bit fields (sign bit 3, exponent bits 2..1, mantissa bit
    0, bias 1); written independently of any table."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if s else mag


def test_e2m1_value_set_is_the_pages_list():
    mags = sorted(float(v) for v in _golden_numbers("e2m1_magnitudes.txt"))
    got = sorted({abs(oracle.e2m1(c)) for c in range(16)})
    assert got == mags
    # every magnitude appears once positive and once negative
    vals = [oracle.e2m1(c) for c in range(16)]
    for m in mags:
        assert vals.count(m) + vals.count(-m) == 2 or m == 0.0


def test_e2m1_exhaustive_vs_bit_formula():
    for c in range(16):
        a, b = oracle.e2m1(c), _ocp_e2m1_from_bits(c)
        assert a == b and np.signbit(a) == np.signbit(b), c
    assert np.signbit(oracle.e2m1(8)) and oracle.e2m1(8) == 0.0  # code 8 is -0


def test_worked_nibble_0b0110():
    # the deep-dive exercise: nibble 0b0110 -> exponent field 3, mantissa 0 -> 4
    assert oracle.e2m1(0b0110) == 4.0
    assert oracle.e2m1(0b1110) == -4.0


def test_e8m0_exhaustive():
    for s in range(255):
        assert oracle.e8m0(s) == 2.0 ** (s - 127)
    # independent check through the fp32 bit pattern: 2^(s-127) has exponent field s
    for s in range(1, 255):
        assert struct.unpack("<f", struct.pack("<I", s << 23))[0] == oracle.e8m0(s)
    assert oracle.e8m0(0) == struct.unpack("<f", struct.pack("<I", 1 << 22))[0]  # fp32 subnormal 2^-127
    assert np.isnan(oracle.e8m0(255))


def test_expert_size_matches_the_pages():
    g = dict(line.split() for line in _golden_numbers("mxfp4_expert_size.txt"))
    params = int(g["params_per_expert"])
    # an expert = three d x f matrices; the oracle consumes codes [rows][cols/2]
    # and scales [rows][cols/32] per matrix -- no padding anywhere
    d, f = 7168, 1536
    assert 3 * d * f == params
    nbytes = 0
    for rows, cols in ((f, d), (f, d), (d, f)):
        codes = np.zeros((rows, cols // 2), np.uint8)
        scales = np.zeros((rows, cols // 32), np.uint8)
        assert oracle.mx_dequant(codes[:2], scales[:2]).shape == (2, cols)
        nbytes += codes.nbytes + scales.nbytes
    assert nbytes == int(g["bytes_per_expert"])
    assert nbytes / params == float(g["bytes_per_param"])
    fp32 = params * 4
    assert round(fp32 / 1e6) == int(g["fp32_megabytes_per_expert"])
    assert int(g["routed_layers"]) * int(g["experts_per_layer_per_token"]) == int(g["experts_per_token"])
    assert round(int(g["experts_per_token"]) * fp32 / 1e9) == int(g["dequant_gigabytes_per_token"])


@pytest.mark.parametrize("pos", [0, 1, 2, 3, 62, 63])
def test_nibble_order_one_hot(pos):
    codes = np.zeros((1, 32), np.uint8)
    scales = np.full((1, 2), 127, np.uint8)
    codes[0, pos // 2] = 0x02 << (4 * (pos % 2))  # code 2 (= 1.0) in element `pos`
    out = oracle.mx_dequant(codes, scales)[0]
    expect = np.zeros(64)
    expect[pos] = 1.0
    assert np.array_equal(out, expect)


def test_scale_applies_per_32_block():
    codes = np.full((1, 32), 0x22, np.uint8)  # every element 1.0
    scales = np.array([[130, 120]], np.uint8)
    out = oracle.mx_dequant(codes, scales)[0]
    assert np.all(out[:32] == 8.0) and np.all(out[32:] == 2.0 ** -7)


def test_dequant_random_vs_bit_decode():
    r = np.random.default_rng(5)
    codes = r.integers(0, 256, (7, 48), dtype=np.uint8)
    scales = r.integers(100, 150, (7, 3), dtype=np.uint8)
    out = oracle.mx_dequant(codes, scales)
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(7, 96)
    ref = np.vectorize(_ocp_e2m1_from_bits)(nib) * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    assert np.array_equal(out, ref)
