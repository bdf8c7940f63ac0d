"""Pins for the oracle's element codecs and shared-exponent rule.

The oracle encodes by searching the decoded grid; these tests check it against
other formulations: the E2M1 rounding thresholds written out as a closed form,
PyTorch's float8_e4m3fn conversion (an independent library routine), the OCP MX
v1.0 grid values, and the defining inequality of the shared exponent.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bits_to_f32

E2M1_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX v1.0, FP4 E2M1


def e2m1_threshold_code(v: float) -> int:
    """Closed-form RNE thresholds on the E2M1 grid (ties to the even code), saturating."""
    m = abs(v)
    if m <= 0.25:
        i = 0
    elif m < 0.75:
        i = 1
    elif m <= 1.25:
        i = 2
    elif m < 1.75:
        i = 3
    elif m <= 2.5:
        i = 4
    elif m < 3.5:
        i = 5
    elif m <= 5.0:
        i = 6
    else:
        i = 7
    return (8 if math.copysign(1.0, v) < 0 else 0) | i


def test_e2m1_decode_grid():
    for c in range(16):
        mag = E2M1_MAGS[c & 7]
        assert oracle.e2m1_decode(c) == (-mag if c & 8 else mag) or (mag == 0 and oracle.e2m1_decode(c) == 0)
        assert math.copysign(1.0, oracle.e2m1_decode(c)) == (-1.0 if c & 8 else 1.0)


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue  # NaN codes
        assert oracle.e4m3_decode(c) == ref[c], c
    assert oracle.e4m3_decode(0x7E) == 448.0


@pytest.mark.parametrize("scale_exp", [0, -3, 5])
def test_e2m1_encode_exhaustive_bf16(scale_exp):
    """Every finite bf16 pattern, divided by 2^scale_exp, against the threshold table."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits_to_f32(bits).astype(np.float64)
    finite = np.isfinite(vals)
    for x in vals[finite][::7]:  # a 1-in-7 stride still visits every exponent and mantissa class
        v = math.ldexp(float(x), -scale_exp)
        assert oracle.e2m1_encode(v) == e2m1_threshold_code(v), v


def test_e2m1_encode_every_tie_and_boundary():
    for v, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
                    (0.2499, 0), (0.2501, 1), (5.0001, 7), (6.0, 7), (7.99, 7), (1e30, 7),
                    (-0.25, 8), (-0.0, 8), (0.0, 0), (-5.5, 15), (-1e-30, 8)]:
        assert oracle.e2m1_encode(v) == code, (v, code)


def test_e4m3_encode_matches_torch_in_range():
    """All finite bf16 magnitudes up to 448 (several scalings) vs torch's RNE conversion."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits_to_f32(bits).astype(np.float64)
    ok = np.isfinite(vals)
    for sh in (0, -20, 12):
        v = np.ldexp(vals[ok], sh)
        v = v[np.abs(v) <= 448.0]
        v32 = torch.from_numpy(v.astype(np.float32))
        ref = v32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = np.array([oracle.e4m3_encode(float(x)) for x in v[::5]], dtype=np.uint8)
        np.testing.assert_array_equal(got, ref[::5])


def test_e4m3_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 511.0, 1e9):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE


def test_roundtrip_every_code_at_many_scales():
    for e in (-127, -40, -2, 0, 3, 100):
        for c in range(16):
            v = math.ldexp(oracle.e2m1_decode(c), e)
            if v == 0 and c == 8:
                v = -0.0
            assert oracle.e2m1_encode(math.ldexp(v, -e)) == c
        for c in range(256):
            if (c & 0x7F) == 0x7F:
                continue
            v = oracle.e4m3_decode(c)
            if c == 0x80:
                v = -0.0
            assert oracle.e4m3_encode(v) == c


@pytest.mark.parametrize("fmt,emax", [(oracle.MXFP4, 2), (oracle.MXFP8, 8)])
def test_scale_exp_definition(fmt, emax):
    rng = np.random.default_rng(7)
    for _ in range(2000):
        amax = math.ldexp(rng.uniform(1.0, 2.0), int(rng.integers(-140, 128)))
        e = oracle.scale_exp(amax, fmt)
        if -127 < e < 127:
            assert 2.0 ** (e + emax) <= amax < 2.0 ** (e + emax + 1)
        else:
            assert e in (-127, 127)
    # special cases
    assert oracle.scale_exp(0.0, fmt) == -127
    assert oracle.scale_exp(4.0, oracle.MXFP4) == 0
    assert oracle.scale_exp(7.99, oracle.MXFP4) == 0
    assert oracle.scale_exp(8.0, oracle.MXFP4) == 1
    assert oracle.scale_exp(256.0, oracle.MXFP8) == 0
    assert oracle.scale_exp(511.0, oracle.MXFP8) == 0
    assert oracle.scale_exp(2.0 ** -133, fmt) == -127        # bf16 subnormal amax
    assert oracle.scale_exp(2.0 ** 127 * 1.5, oracle.MXFP4) == 125
