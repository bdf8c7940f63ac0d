"""Pins for the oracle's activation quantization with outlier extraction and its weight packing.

Checks against: the hand-worked G=32 group in tests/golden (derived from the OSC
page §3.2 and the OCP MX v1.0 rules), the exact-rational restatement in
tests/exact_ref.py, and invariants the page fixes (B holds the indexed value
bit for bit; the zeroed slot encodes as +0; the scale is computed on the
zeroed group; with no table entry the path is plain MX quantization).
"""
import json
import os

import numpy as np
import pytest

import oracle
import exact_ref
from synth import bits_to_f32, random_bf16, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_group_g32.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_group_osc_and_direct():
    g = _golden()
    x = to_bf16_bits(np.array([g["x_values"]], np.float32))
    # with OSC extraction
    QX, SX, B = oracle.quant_act(x, 32, np.array([g["osc"]["L"]], np.int32))
    assert [f"{b:02X}" for b in QX[0]] == g["osc"]["packed_bytes"]
    assert SX[0, 0] == g["osc"]["scale_code"]
    assert B[0, 0] == int(g["osc"]["B_bits"], 16)
    # direct MXFP4, with no table entry
    QXd, SXd, Bd = oracle.quant_act(x, 32, np.array([-1], np.int32))
    assert [f"{b:02X}" for b in QXd[0]] == g["direct"]["packed_bytes"]
    assert SXd[0, 0] == g["direct"]["scale_code"]
    assert Bd[0, 0] == 0
    # weights of all ones
    w = to_bf16_bits(np.ones((1, 32), np.float32))
    QW, SW, WL = oracle.pack_weights(w, 32, np.array([g["osc"]["L"]], np.int32))
    assert SW[0, 0] == g["weight_all_ones"]["scale_code"]
    assert all(b == 0x66 for b in QW[0])
    assert WL[0, 0] == to_bf16_bits(np.array([1.0], np.float32))[0]
    # dual-path outputs
    Y = oracle.gemm(QX, SX, QW, SW, 32, B, WL)
    assert Y[0, 0] == g["Y"]["osc"]
    QWd, SWd, _ = oracle.pack_weights(w, 32, None)
    assert oracle.gemm(QXd, SXd, QWd, SWd, 32)[0, 0] == g["Y"]["direct"]


@pytest.mark.parametrize("G", [16, 32, 64])
@pytest.mark.parametrize("fp8", [False, True])
def test_quant_matches_exact_rationals(G, fp8):
    S, H = 3, 128
    X = random_bf16((S, H), seed=G + 100 * fp8, scale=2.0)
    X[1, 5] = 0x8000          # a -0 input
    X[2, G:2 * G] = 0          # an all-zero group
    X[0, 3] = to_bf16_bits(np.array([3e-39], np.float32))[0]  # a bf16 subnormal
    rng = np.random.default_rng(G)
    L = None if fp8 else rng.integers(-1, G, H // G).astype(np.int32)
    fmt = oracle.MXFP8 if fp8 else oracle.MXFP4
    QX, SX, B = oracle.quant_act(X, G, L, fmt)
    codes, exps, bvals = exact_ref.quant_rows(X.tolist(), G, None if L is None else L.tolist(), fp8)
    for s in range(S):
        for k in range(H // G):
            assert SX[s, k] == exps[s][k] + 127
            if L is not None:
                assert B[s, k] == bvals[s][k]
        for h in range(H):
            got = QX[s, h] if fp8 else (QX[s, h // 2] >> (4 * (h % 2))) & 0xF
            assert got == codes[s][h], (s, h)


def test_extraction_invariants_at_scale():
    S, H, G = 64, 512, 32
    X = random_bf16((S, H), seed=3)
    rng = np.random.default_rng(4)
    L = rng.integers(-1, G, H // G).astype(np.int32)
    QX, SX, B = oracle.quant_act(X, G, L)
    xv = bits_to_f32(X).astype(np.float64)
    for k in range(H // G):
        c = L[k]
        if c >= 0:
            np.testing.assert_array_equal(B[:, k], X[:, k * G + c])
            col = k * G + c
            nib = (QX[:, col // 2] >> (4 * (col % 2))) & 0xF
            assert np.all(nib == 0)  # zeroed slot encodes as +0
        else:
            assert np.all(B[:, k] == 0)
        # scale on the zeroed group, by an independent computation
        g = np.abs(xv[:, k * G:(k + 1) * G]).copy()
        if c >= 0:
            g[:, c] = 0
        amax = g.max(axis=1)
        _, p = np.frexp(amax)
        e = np.where(amax > 0, np.clip(p - 1 - 2, -127, 127), -127)
        np.testing.assert_array_equal(SX[:, k].astype(np.int64), e + 127)


def test_no_table_entry_is_plain_mx():
    X = random_bf16((8, 256), seed=9)
    QX1, SX1, B1 = oracle.quant_act(X, 32, np.full(8, -1, np.int32))
    QX2, SX2, _ = oracle.quant_act(X, 32, None)
    np.testing.assert_array_equal(QX1, QX2)
    np.testing.assert_array_equal(SX1, SX2)
    assert np.all(B1 == 0)


def test_pack_weights_layout():
    N, H, G = 5, 128, 32
    W = random_bf16((N, H), seed=5, scale=0.02)
    L = np.array([3, -1, 0, 31], np.int32)
    QW, SW, WL = oracle.pack_weights(W, G, L)
    QX, SX, _ = oracle.quant_act(W, G, None)  # the weight side is plain MX quantization of W
    np.testing.assert_array_equal(QW, QX)
    np.testing.assert_array_equal(SW, SX)
    for k in range(4):
        if L[k] >= 0:
            np.testing.assert_array_equal(WL[:, k], W[:, k * G + L[k]])
        else:
            assert np.all(WL[:, k] == 0)
