"""Pins of the oracle's E3M2-pair encoding of G = 16 (the fast-G=16 item: two 16-groups of an
MXFP4 G = 16 quantization carried by one E8M0 scale and 32 E3M2 codes, so the matrix cores' 32-wide
scale blocks run G = 16 at the FP4 issue rate; OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署",
§3.3 Table 2 and §6).

Pinned by: the OCP E3M2 grid's defining facts (bias 3, 28 largest, 1/16 smallest, 31 distinct
magnitudes, monotone, sign bit 5) and round trips; ties to even; reduction to the single-group
G = 16 MXFP4 oracle -- every decoded E3M2 value times its pair scale equals the MXFP4 value times its
group scale, and the whole GEMM equals the G = 16 OSC GEMM in fp64, whenever the two groups' scale
codes differ by at most 5; a hand-built pair with a gap of 7 whose smaller group rounds."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from synth import to_bf16_bits


def test_e3m2_grid():
    mags = [oracle.e3m2_decode(c) for c in range(32)]
    assert mags[0] == 0.0 and mags[1] == 1 / 16 and mags[31] == 28.0
    assert mags[4] == 0.25                      # smallest normal: 2^(1-3)
    assert all(a < b for a, b in zip(mags, mags[1:]))
    for c in range(32):
        assert oracle.e3m2_decode(c | 32) == -mags[c]
        v = Fraction(mags[c])
        if c >= 4:
            # a normal value: 2^e * (1 + m/4) with e in [-2, 4] and a 2-bit mantissa m
            e = math.floor(math.log2(mags[c]))
            f = v / Fraction(2) ** e
            assert -2 <= e <= 4 and 1 <= f < 2 and (4 * f).denominator == 1
        else:
            assert v == Fraction(c, 16)  # subnormals: multiples of 1/16


def test_e3m2_encode_round_trip_ties_and_saturation():
    for c in range(64):
        if c == 32:
            continue  # -0 encodes as -0 only from a negative zero
        assert oracle.e3m2_encode(oracle.e3m2_decode(c)) == c
    assert oracle.e3m2_encode(-0.0) == 32
    assert oracle.e3m2_encode(1.5 / 16) == 2     # tie between 1/16 and 2/16: even code
    assert oracle.e3m2_encode(0.5 / 16) == 0     # tie between 0 and 1/16
    assert oracle.e3m2_encode(1.125) == 12       # tie between 1 and 1.25: even mantissa (1.0)
    assert oracle.e3m2_encode(1.375) == 14       # tie between 1.25 and 1.5: even (1.5)
    assert oracle.e3m2_encode(100.0) == 31 and oracle.e3m2_encode(-30.0) == 63


def _pairs_within_gap(Q4S16, gap=5):
    s = Q4S16.astype(int)
    return np.all(np.abs(s[:, 0::2] - s[:, 1::2]) <= gap)


def test_pairs_reduce_to_the_g16_values_elementwise():
    S, H = 24, 512
    X = synth.random_bf16((S, H), seed=3, scale=2.0)
    L = np.random.default_rng(4).integers(-1, 16, H // 16).astype(np.int32)
    q4, s16, b4 = oracle.quant_act_multi(X, 16, L.reshape(-1, 1), 1)
    assert _pairs_within_gap(s16)
    q6, s32, b6 = oracle.quant_act_fp6p(X, L, 1)
    np.testing.assert_array_equal(b6, b4)
    for k in range(H):
        v4 = np.array([oracle.e2m1_decode(int((q4[s, k // 2] >> (4 * (k % 2))) & 15)) for s in range(S)])
        v4 = v4 * np.exp2(s16[:, k // 16].astype(float) - 127)
        c6 = oracle.get_code6(q6, k)
        v6 = np.array([oracle.e3m2_decode(int(c)) for c in c6]) * np.exp2(s32[:, k // 32].astype(float) - 127)
        np.testing.assert_array_equal(v6, v4)
    # the pair scale: the larger group's code minus 2, at least 0
    np.testing.assert_array_equal(s32.astype(int), np.maximum(np.maximum(s16[:, 0::2], s16[:, 1::2]).astype(int) - 2, 0))


def test_pairs_gemm_equals_the_g16_osc_gemm():
    S, N, H = 12, 20, 256
    X = synth.random_bf16((S, H), seed=5, scale=3.0)
    W = synth.random_bf16((N, H), seed=6, scale=0.05)
    L = np.random.default_rng(7).integers(-1, 16, H // 16).astype(np.int32)
    y16 = oracle.osc_linear(X, W, 16, L)
    q6x, s32x, b = oracle.quant_act_fp6p(X, L, 1)
    q6w, s32w, wl = oracle.pack_weights_fp6p(W, L, 1)
    np.testing.assert_array_equal(oracle.gemm_fp6p(q6x, s32x, q6w, s32w, b, wl), y16)
    # no table: the plain G = 16 MXFP4 product
    q6x, s32x, _ = oracle.quant_act_fp6p(X)
    q6w, s32w, _ = oracle.pack_weights_fp6p(W)
    np.testing.assert_array_equal(oracle.gemm_fp6p(q6x, s32x, q6w, s32w), oracle.osc_linear(X, W, 16, None))


def test_pair_with_a_gap_of_seven_rounds_the_smaller_group():
    """Group 0: amax 64 (E8M0 code 133 - 2 = 131); group 1: amax 0.75 (code 126 - 2 = 124): E = 129,
    the smaller group's values are scaled by 2^-5.  0.75 -> E2M1 6 at 2^-3 -> 6 * 2^-5 = 3/16 (exact);
    0.0625 -> E2M1 0.5 -> 2^-6 = 0.25/16 -> rounds to 0; 0.25 -> 2 -> 1/16 (exact)."""
    row = np.zeros(32)
    row[0] = 64.0
    row[16] = 0.75
    row[17] = 0.0625
    row[18] = -0.25
    X = to_bf16_bits(row.reshape(1, 32).repeat(1, 0))
    X = np.concatenate([X, np.zeros((1, 224), np.uint16)], axis=1)  # H = 256
    q6, s32, _ = oracle.quant_act_fp6p(X)
    assert int(s32[0, 0]) == 129
    assert oracle.e3m2_decode(int(oracle.get_code6(q6, 0)[0])) == 16.0      # 64 = 16 * 2^(129-127)
    assert oracle.get_code6(q6, 16)[0] == 3                               # 3/16
    assert oracle.get_code6(q6, 17)[0] == 0                               # 1/64 rounds to 0
    assert oracle.get_code6(q6, 18)[0] == 32 | 1                          # -1/16
    q4, s16, _ = oracle.quant_act(X, 16, None)
    assert (int(s16[0, 0]), int(s16[0, 1])) == (131, 124)
