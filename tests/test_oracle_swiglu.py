"""Pins of the oracle's MLP glue (h = silu(gate) * up, the input of a Qwen3-shaped block's
down-projection W2) and of the clustering-density average behind §2.3's per-module rule (OSC page
"W4A4量化技术：OSC框架如何实现高效LLM部署", §2.2 / §2.3).

The glue is defined as binary32 operations (Cody-Waite exp, correctly rounded division, bf16
round-to-nearest-even) so the device can match it bit for bit; here it is pinned against the
mathematics: fp64 exp and silu within a few binary32 ulps, the limits where 1 + e^-g rounds to 1,
signed zeros, exact products, and bf16 rounding checked with exact rationals."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import bits_to_f32, to_bf16_bits


def f32(x):
    return float(np.float32(x))


def test_exp32_within_four_ulps_of_exp():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.uniform(-86.0, 88.0, 4000), np.linspace(-1, 1, 513), [0.0, 1e-30, -1e-30]])
    for x in xs.astype(np.float32):
        got = oracle.exp32(float(x))
        ref = math.exp(float(x))
        ulp = math.ldexp(1.0, math.frexp(ref)[1] - 24)
        assert abs(got - ref) <= 4 * ulp, (float(x), got, ref)


def test_exp32_limits():
    assert oracle.exp32(0.0) == 1.0
    assert oracle.exp32(88.0) < math.inf and oracle.exp32(88.0 + 2 ** -17) == math.inf
    assert oracle.exp32(-86.0) > 0.0 and oracle.exp32(-86.0 - 2 ** -17) == 0.0
    assert oracle.exp32(-86.0) >= 2.0 ** -126  # every finite result is a normal number


def test_silu32_against_fp64():
    rng = np.random.default_rng(2)
    gs = np.concatenate([rng.normal(0, 3, 3000), rng.uniform(-80, 80, 1000)]).astype(np.float32)
    for g in gs:
        g = float(g)
        ref = g / (1.0 + math.exp(-g))
        got = oracle.silu32(g)
        ulp = math.ldexp(1.0, math.frexp(ref)[1] - 24) if ref != 0 else 2.0 ** -149
        assert abs(got - ref) <= 6 * ulp, (g, got, ref)


def test_silu32_special_values():
    assert oracle.silu32(0.0) == 0.0 and math.copysign(1.0, oracle.silu32(-0.0)) == -1.0
    for g in (87.0, 100.0, 1e4, 3.0e38):  # 1 + e^-g rounds to 1: silu(g) = g exactly
        assert oracle.silu32(g) == f32(g)
    for g in (-88.5, -1e4, -3.0e38):        # e^-g beyond the binary32 range: the quotient is -0
        v = oracle.silu32(g)
        assert v == 0.0 and math.copysign(1.0, v) == -1.0
    assert oracle.silu32(-88.0) < 0.0       # still a (tiny) normal quotient at the edge


def _exact_bf16_rne(x: float) -> int:
    """bf16 rounding of a finite binary32 value with exact rationals (ties to even)."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    a = Fraction(abs(x))
    e = math.floor(math.log2(abs(x)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = a / Fraction(2) ** (e - 7)          # 8 significant bits (subnormals: fixed exponent)
    n = math.floor(q)
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = Fraction(n) * Fraction(2) ** (e - 7)
    return sign | int(to_bf16_bits(np.array([float(v)], np.float64))[0])


def test_bf16_rne_exact_and_ties():
    assert oracle.bf16_rne(1.0 + 2 ** -8) == 0x3F80           # tie between 1 and 1+2^-7: even (1)
    assert oracle.bf16_rne(1.0 + 3 * 2 ** -8) == 0x3F82       # tie between 1+2^-7 and 1+2^-6: even
    assert oracle.bf16_rne(-(1.0 + 2 ** -8 + 2 ** -20)) == 0xBF81
    rng = np.random.default_rng(3)
    for x in np.concatenate([rng.normal(0, 1, 300), rng.normal(0, 1e-30, 50), rng.normal(0, 1e30, 50)]).astype(np.float32):
        assert oracle.bf16_rne(float(x)) == _exact_bf16_rne(float(x)), float(x)


def test_swiglu_within_bf16_rounding_of_fp64():
    rng = np.random.default_rng(4)
    S, F = 6, 256
    g = to_bf16_bits(rng.normal(0, 2.0, (S, F)))
    u = to_bf16_bits(rng.normal(0, 1.0, (S, F)))
    Hh = oracle.swiglu(np.concatenate([g, u], axis=1))
    gv, uv = bits_to_f32(g).astype(np.float64), bits_to_f32(u).astype(np.float64)
    ref = gv / (1.0 + np.exp(-gv)) * uv
    got = bits_to_f32(Hh).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) * 1.0001 + 1e-37)


def test_swiglu_exact_cases():
    S, F = 2, 256
    g = np.zeros((S, F), np.float64)
    u = np.zeros((S, F), np.float64)
    g[0, :] = np.linspace(87, 300, F)        # silu(g) = g exactly in binary32
    u[0, :] = 2.0 ** (np.arange(F) % 7)      # u in {1, 2, 4, ..., 64}: exact products
    g[1, :] = np.linspace(-5, 5, F)
    u[1, :] = 0.0                            # zero up: h = +-0
    gb, ub = to_bf16_bits(g), to_bf16_bits(u)
    Hh = oracle.swiglu(np.concatenate([gb, ub], axis=1))
    prod = bits_to_f32(gb[0]).astype(np.float64) * bits_to_f32(ub[0]).astype(np.float64)
    np.testing.assert_array_equal(bits_to_f32(Hh[0]).astype(np.float64), prod)
    assert np.all((Hh[1] & 0x7FFF) == 0)


def test_swiglu_quant_is_quantization_of_h():
    rng = np.random.default_rng(5)
    S, F, G = 5, 512, 32
    GU = to_bf16_bits(rng.normal(0, 1.5, (S, 2 * F)))
    Hh = oracle.swiglu(GU)
    for fmt in (oracle.MXFP4, oracle.MXFP8):
        for a, b in zip(oracle.swiglu_quant(GU, G, None, 1, fmt), oracle.quant_act(Hh, G, None, fmt)):
            np.testing.assert_array_equal(a, b)
    L = np.array([[3], [-1], [7], [31]] * 4, np.int32)
    for a, b in zip(oracle.swiglu_quant(GU, G, L, 1), oracle.quant_act_multi(Hh, G, L, 1)):
        np.testing.assert_array_equal(a, b)


def test_mean_density_hand_values():
    hits = np.array([3, 0, 5, 9], np.int32)
    events = np.array([4, 0, 10, 9], np.int32)
    assert oracle.mean_density(hits, events) == pytest.approx((0.75 + 0.5 + 1.0) / 3)
    assert oracle.mean_density(np.zeros(3, np.int32), np.zeros(3, np.int32)) == 0.0
    # several entries per group: the first (kept) entry's count is the group's N_hit
    hm = np.array([[3, 1], [2, 2]], np.int32)
    assert oracle.mean_density(hm, np.array([4, 8], np.int32)) == pytest.approx((0.75 + 0.25) / 2)


def test_mean_density_of_built_tables_separates_the_workloads():
    """On the seeded workloads the persistent-channel recipe (QKV) clusters far above the 35 % line
    and the diffuse-spike recipe of W2 (one spike per token at a random channel in 288 of 384
    groups) far below it, the split §2.3's rule is meant to detect."""
    import synth
    q = synth.qkv(S=16)
    L, hits, ev = oracle.build_table(q.calib, 32)
    assert oracle.mean_density(hits, ev) >= 0.6
    d = synth.ffn_down(S=16)
    L, hits, ev = oracle.build_table(d.calib, 32)
    assert oracle.mean_density(hits, ev) < 0.35
