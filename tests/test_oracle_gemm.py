"""Pins for the oracle's dual-path GEMM (OSC page §3.2; FP8 fallback §4).

* brute force: the exact-rational restatement in tests/exact_ref.py on tiny shapes;
* two-path identity: when every residual element already lies on the E2M1 grid at
  its group's scale and W is MXFP4-exact, Y equals the plain product X·Wᵀ exactly;
* power-of-two equivariance and sign symmetry.
"""
import numpy as np
import pytest

import oracle
import exact_ref
from synth import bits_to_f32, random_bf16, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.mark.parametrize("G", [16, 32, 64])
@pytest.mark.parametrize("mode", ["osc", "direct", "fp8_w4", "fp8_w8"])
def test_gemm_matches_exact_rationals(G, mode):
    S, N, H = 3, 4, 128
    seed = G * 10 + len(mode)
    X = random_bf16((S, H), seed=seed, scale=1.0)
    rng = np.random.default_rng(seed)
    # plant some large channels so that extraction matters
    for k in range(H // G):
        X[:, k * G + (k * 7) % G] = to_bf16_bits(bits_to_f32(X[:, k * G + (k * 7) % G]) * 60.0)
    W = random_bf16((N, H), seed=seed + 1, scale=0.02)
    L = rng.integers(-1, G, H // G).astype(np.int32)
    if mode == "osc":
        Y = oracle.osc_linear(X, W, G, L)
        Yx = exact_ref.osc_linear(X.tolist(), W.tolist(), G, L.tolist())
    elif mode == "direct":
        QX, SX, _ = oracle.quant_act(X, G, None)
        QW, SW, _ = oracle.pack_weights(W, G, None)
        Y = oracle.gemm(QX, SX, QW, SW, G)
        Yx = exact_ref.osc_linear(X.tolist(), W.tolist(), G, None)
    else:
        wfmt = oracle.MXFP8 if mode == "fp8_w8" else oracle.MXFP4
        QX, SX, _ = oracle.quant_act(X, G, None, oracle.MXFP8)
        QW, SW, _ = oracle.pack_weights(W, G, None, wfmt)
        Y = oracle.gemm(QX, SX, QW, SW, G, afmt=oracle.MXFP8, wfmt=wfmt)
        Yx = exact_ref.osc_linear(X.tolist(), W.tolist(), G, None, act_fp8=True, w_fp8=(mode == "fp8_w8"))
    for s in range(S):
        for n in range(N):
            # every product is exact in fp64 and the sums of these dyadic values stay exact
            assert Y[s, n] == float(Yx[s][n]), (s, n, Y[s, n], float(Yx[s][n]))


def _mx_exact_rows(rng, rows, H, G, e_lo, e_hi):
    """Rows whose every G-group is exactly representable in MXFP4 (some element of magnitude 4 or 6)."""
    out = np.zeros((rows, H))
    for r in range(rows):
        for k in range(H // G):
            e = int(rng.integers(e_lo, e_hi + 1))
            idx = rng.integers(0, 8, G)
            idx[rng.integers(0, G)] = rng.choice([6, 7])
            sign = rng.choice([-1.0, 1.0], G)
            out[r, k * G:(k + 1) * G] = sign * GRID[idx] * 2.0 ** e
    return out


@pytest.mark.parametrize("G", [16, 32, 64])
def test_two_path_identity_is_exact(G):
    S, N, H = 6, 7, 256
    rng = np.random.default_rng(G)
    xr = _mx_exact_rows(rng, S, H, G, -3, 3)
    L = rng.integers(-1, G, H // G).astype(np.int32)
    for k in range(H // G):
        if L[k] >= 0:  # the extracted slot carries an arbitrary large bf16 value
            xr[:, k * G + L[k]] = bits_to_f32(to_bf16_bits(rng.normal(0, 80.0, S)))
    w = _mx_exact_rows(rng, N, H, G, -9, -5)
    X = to_bf16_bits(xr)
    W = to_bf16_bits(w)
    assert np.array_equal(bits_to_f32(X).astype(np.float64), xr)
    Y = oracle.osc_linear(X, W, G, L)
    np.testing.assert_array_equal(Y, xr @ w.T)


def test_power_of_two_equivariance_and_sign_symmetry():
    S, N, H, G = 5, 6, 256, 32
    X = random_bf16((S, H), seed=21)
    W = random_bf16((N, H), seed=22, scale=0.02)
    L = np.random.default_rng(23).integers(-1, G, H // G).astype(np.int32)
    QX, SX, B = oracle.quant_act(X, G, L)
    Y = oracle.osc_linear(X, W, G, L)
    X8 = to_bf16_bits(bits_to_f32(X) * 8.0)
    QX8, SX8, _ = oracle.quant_act(X8, G, L)
    np.testing.assert_array_equal(QX8, QX)
    np.testing.assert_array_equal(SX8.astype(int), SX.astype(int) + 3)
    np.testing.assert_array_equal(oracle.osc_linear(X8, W, G, L), Y * 8.0)
    Xn = X ^ np.uint16(0x8000)
    np.testing.assert_array_equal(oracle.osc_linear(Xn, W, G, L), -Y)
