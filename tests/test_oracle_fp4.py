"""Pins of the oracle's MXFP4 codec (fp4 indexer cache, reading R25) against the format definition.

OCP Microscaling Formats v1.0: e2m1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit; the
exponent-0 codes are 0 and 0.5), one E8M0 scale 2^X per 32 elements with X = floor(log2 amax) - 2.
Expected values below are written out by hand from that definition, not produced by the oracle.
"""
import numpy as np
import pytest

from oracle import codecs

# code -> value, from the bit layout s.ee.m: (-1)^s * (e ? 2^(e-1) * (1 + m/2) : m/2)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_decode_table():
    got = codecs.e2m1_to_f64(np.arange(16))
    assert got.tolist() == E2M1_TABLE
    assert np.signbit(got[8])


def test_e2m1_encode_representable_values_round_trip():
    for code, v in enumerate(E2M1_TABLE):
        if code == 8:
            continue  # -0.0 is not negative: encodes as +0
        assert int(codecs.f64_to_e2m1(v)) == code


@pytest.mark.parametrize("x,code", [
    (0.25, 0),   # tie 0 | 0.5 -> even code 0
    (0.75, 2),   # tie 0.5 | 1 -> code 2
    (1.25, 2),   # tie 1 | 1.5 -> code 2
    (1.75, 4),   # tie 1.5 | 2 -> code 4
    (2.5, 4),    # tie 2 | 3 -> code 4
    (3.5, 6),    # tie 3 | 4 -> code 6
    (5.0, 6),    # tie 4 | 6 -> code 6
    (0.2500001, 1), (0.7499999, 1), (4.9999, 6), (5.0001, 7),
    (6.5, 7), (1e9, 7),                  # saturation at 6
    (-5.0, 14), (-0.1, 8), (-7.0, 15),  # sign bit set for every negative input
])
def test_e2m1_ties_and_saturation(x, code):
    assert int(codecs.f64_to_e2m1(x)) == code


def test_e2m1_nearest_brute_force():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-6, 6, 20000), np.arange(-24, 25) / 4.0])
    codes = codecs.f64_to_e2m1(x)
    mags = np.array(E2M1_TABLE[:8])
    for xi, c in zip(x, codes):
        d = np.abs(abs(xi) - mags)
        assert d[c & 7] == d.min()
        if np.count_nonzero(d == d.min()) == 2:
            assert (c & 1) == 0


def test_mx_block_exponent():
    assert codecs.mx_block_exponent(6.0) == 0       # floor(log2 6) = 2
    assert codecs.mx_block_exponent(4.0) == 0
    assert codecs.mx_block_exponent(3.99) == -1
    assert codecs.mx_block_exponent(1.0) == -2
    assert codecs.mx_block_exponent(0.0) == 0
    assert codecs.mx_block_exponent(2.0 ** -140) == -127  # clamped to the E8M0 range
    assert codecs.mx_block_exponent(2.0 ** 127) == 125


def test_mxfp4_worked_block():
    # block 0: amax 3 -> X = -1, elements y / 0.5; block 1: all zero -> X = 0, codes 0
    y = np.zeros(64, dtype=np.float32)
    y[0:6] = [3.0, -3.0, 0.25, 0.2, 1.3, -0.7]
    packed, exps = codecs.f32_to_mxfp4(y)
    assert exps.tolist() == [126, 127]
    # y / 0.5 = 6, -6, 0.5, 0.4 -> 0.5, 2.6 -> 3, -1.4 -> -1.5
    assert packed[:3].tolist() == [0x7 | (0xF << 4), 0x1 | (0x1 << 4), 0x5 | (0xB << 4)]
    assert not packed[16:].any()
    back = codecs.mxfp4_to_f64(packed, exps)
    assert back[:6].tolist() == [3.0, -3.0, 0.25, 0.25, 1.5, -0.75]
    assert not back[6:].any()


def test_mxfp4_saturates_above_six_steps():
    # amax 7 -> X = floor(log2 7) - 2 = 0: 7 saturates to 6 (the format's known clipping)
    y = np.full(32, 0.5, dtype=np.float32)
    y[3] = 7.0
    packed, exps = codecs.f32_to_mxfp4(y)
    assert exps.tolist() == [127]
    assert codecs.mxfp4_to_f64(packed, exps)[3] == 6.0


def test_mxfp4_error_bound():
    rng = np.random.default_rng(9)
    for _ in range(200):
        y = (rng.standard_normal(128) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        packed, exps = codecs.f32_to_mxfp4(y)
        back = codecs.mxfp4_to_f64(packed, exps)
        for b in range(4):
            blk = y[32 * b:32 * b + 32].astype(np.float64)
            X = int(exps[b]) - 127
            v = np.abs(blk) / 2.0 ** X
            half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))  # half the e2m1 spacing at |v|
            err = np.abs(back[32 * b:32 * b + 32] - blk) / 2.0 ** X
            ok = np.where(v <= 6, err <= half, err == v - 6)
            assert ok.all()
        assert np.array_equal(back, codecs.mxfp4_to_f64(*codecs.f32_to_mxfp4(back.astype(np.float32))))
