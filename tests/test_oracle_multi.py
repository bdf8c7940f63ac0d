"""Pins of the oracle's several-channels-per-group functions (the §6 direction of the OSC page
"W4A4量化技术：OSC框架如何实现高效LLM部署": protect 2-3 channels per group).

Reading (the page gives only the direction): the table holds m distinct offsets (or -1) per group;
every listed channel goes to its own column of B (group-major, column k*m + j) and is zeroed; the
scale is taken on the group with all of them zeroed; W_L has the same columns; the compensation
is B·W_L over the m*K columns.  Pinned by: reduction to the single-channel functions at m = 1,
an exact-rational restatement (tests/exact_ref.py), invariants checked by an independent numpy
computation, the two-path identity, and hand-built calibration groups for the table builder.
"""
import numpy as np
import pytest

import exact_ref
import oracle
import synth
from synth import bits_to_f32, random_bf16, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def random_multi_table(rng, K, G, m, p_none=0.25):
    """m distinct offsets per group, each replaced by -1 with probability p_none."""
    L = np.full((K, m), -1, np.int32)
    for k in range(K):
        ch = rng.choice(G, size=m, replace=False)
        keep = rng.random(m) >= p_none
        L[k] = np.where(keep, ch, -1)
    return L


# ------------------------------------------------------------------ m = 1

def test_m1_is_the_single_channel_path():
    w = synth.tiny()
    L1 = w.L
    for a, b in zip(oracle.quant_act(w.X, w.G, L1), oracle.quant_act_multi(w.X, w.G, L1.reshape(-1, 1), 1)):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(oracle.pack_weights(w.W, w.G, L1), oracle.pack_weights_multi(w.W, w.G, L1.reshape(-1, 1), 1)):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(oracle.osc_linear(w.X, w.W, w.G, L1),
                                  oracle.osc_linear_multi(w.X, w.W, w.G, L1.reshape(-1, 1), 1))


def test_m1_table_builder_is_the_single_channel_builder():
    q = synth.qkv(S=16)
    cal = q.calib[:512]
    L, hits, ev = oracle.build_table(cal, 32)
    Lm, hm, evm = oracle.build_table_multi(cal, 32, 1)
    np.testing.assert_array_equal(Lm[:, 0], L)
    np.testing.assert_array_equal(hm[:, 0], hits)
    np.testing.assert_array_equal(evm, ev)


# ------------------------------------------------------------------ exact rationals

@pytest.mark.parametrize("G,m", [(16, 2), (32, 2), (32, 3), (64, 3)])
def test_multi_quant_matches_exact_rationals(G, m):
    S, H = 3, 128
    rng = np.random.default_rng(G * 10 + m)
    X = random_bf16((S, H), seed=G + m, scale=4.0)
    L = random_multi_table(rng, H // G, G, m)
    QX, SX, B = oracle.quant_act_multi(X, G, L, m)
    codes, exps, bvals = exact_ref.quant_rows(X.tolist(), G, L.tolist(), False)
    for s in range(S):
        assert [int(v) - 127 for v in SX[s]] == exps[s]
        assert B[s].tolist() == bvals[s]
        for h in range(H):
            assert (QX[s, h // 2] >> (4 * (h % 2))) & 0xF == codes[s][h], (s, h)


@pytest.mark.parametrize("G,m", [(32, 2), (16, 3)])
def test_multi_gemm_matches_exact_rationals(G, m):
    S, N, H = 3, 4, 128
    rng = np.random.default_rng(100 + G + m)
    X = random_bf16((S, H), seed=7 + m, scale=3.0)
    W = random_bf16((N, H), seed=8 + m, scale=0.05)
    L = random_multi_table(rng, H // G, G, m)
    Y = oracle.osc_linear_multi(X, W, G, L, m)
    Yx = exact_ref.osc_linear(X.tolist(), W.tolist(), G, L.tolist())
    for s in range(S):
        for n in range(N):
            assert Y[s, n] == float(Yx[s][n]), (s, n)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("m", [2, 3])
def test_multi_extraction_invariants_at_scale(m):
    S, H, G = 48, 512, 32
    X = random_bf16((S, H), seed=30 + m)
    L = random_multi_table(np.random.default_rng(31 + m), H // G, G, m)
    QX, SX, B = oracle.quant_act_multi(X, G, L, m)
    xv = bits_to_f32(X).astype(np.float64)
    for k in range(H // G):
        g = np.abs(xv[:, k * G:(k + 1) * G]).copy()
        for j in range(m):
            c = L[k, j]
            col = k * m + j
            if c >= 0:
                np.testing.assert_array_equal(B[:, col], X[:, k * G + c])
                h = k * G + c
                assert np.all(((QX[:, h // 2] >> (4 * (h % 2))) & 0xF) == 0)  # zeroed slot -> +0
                g[:, c] = 0
            else:
                assert np.all(B[:, col] == 0)
        amax = g.max(axis=1)
        _, p = np.frexp(amax)
        e = np.where(amax > 0, np.clip(p - 1 - 2, -127, 127), -127)
        np.testing.assert_array_equal(SX[:, k].astype(np.int64), e + 127)


def test_multi_weights_layout():
    N, H, G, m = 20, 256, 32, 2
    W = random_bf16((N, H), seed=41, scale=0.05)
    L = random_multi_table(np.random.default_rng(42), H // G, G, m)
    QW, SW, WL = oracle.pack_weights_multi(W, G, L, m)
    QW1, SW1, _ = oracle.pack_weights(W, G, None)
    np.testing.assert_array_equal(QW, QW1)  # W is quantized unmodified
    np.testing.assert_array_equal(SW, SW1)
    for k in range(H // G):
        for j in range(m):
            want = W[:, k * G + L[k, j]] if L[k, j] >= 0 else np.zeros(N, np.uint16)
            np.testing.assert_array_equal(WL[:, k * m + j], want)


def _mx_exact_rows(rng, rows, H, G, e_lo, e_hi):
    out = np.zeros((rows, H))
    for r in range(rows):
        for k in range(H // G):
            e = int(rng.integers(e_lo, e_hi + 1))
            idx = rng.integers(0, 8, G)
            idx[rng.integers(0, G)] = rng.choice([6, 7])
            sign = rng.choice([-1.0, 1.0], G)
            out[r, k * G:(k + 1) * G] = sign * GRID[idx] * 2.0 ** e
    return out


@pytest.mark.parametrize("G,m", [(32, 2), (64, 3)])
def test_multi_two_path_identity_is_exact(G, m):
    """Y = X·Wᵀ exactly when the activations left after zeroing the m listed channels are
    MXFP4-exact at their group scale and W is MXFP4-exact: the listed channels then travel whole
    through the 16-bit path, whatever their magnitude."""
    S, N, H = 5, 6, 256
    rng = np.random.default_rng(7 * G + m)
    L = np.stack([rng.choice(G, size=m, replace=False) for _ in range(H // G)]).astype(np.int32)
    xr = _mx_exact_rows(rng, S, H, G, -3, 3)
    for k in range(H // G):
        for j in range(m):
            c = L[k, j]
            xr[:, k * G + c] = bits_to_f32(to_bf16_bits(rng.normal(0, 90.0, S)))
    # the residual must still hold a largest element of magnitude 4 or 6 at the group's scale
    for r in range(S):
        for k in range(H // G):
            g = xr[r, k * G:(k + 1) * G].copy()
            g[L[k]] = 0
            if np.abs(g).max() == 0:
                xr[r, k * G + next(c for c in range(G) if c not in L[k])] = 4.0
    w = _mx_exact_rows(rng, N, H, G, -9, -5)
    X = to_bf16_bits(xr)
    W = to_bf16_bits(w)
    assert np.array_equal(bits_to_f32(X).astype(np.float64), xr)
    resid = xr.copy()
    for k in range(H // G):
        resid[:, k * G + L[k]] = 0
    # the residual's own quantization must be exact for the identity to hold
    QX, SX, B = oracle.quant_act_multi(X, G, L, m)
    deq = np.zeros_like(resid)
    for s in range(S):
        for h in range(H):
            code = (QX[s, h // 2] >> (4 * (h % 2))) & 0xF
            deq[s, h] = (-1 if code & 8 else 1) * GRID[code & 7] * 2.0 ** (int(SX[s, h // G]) - 127)
    assert np.array_equal(deq, resid), "the seeded residual must be MXFP4-exact for the identity to apply"
    np.testing.assert_array_equal(oracle.osc_linear_multi(X, W, G, L, m), xr @ w.T)


# ------------------------------------------------------------------ table builder

def _group_rows(R, G, rng, spikes):
    """R calibration rows of one group: N(0,1) background, spikes = [(channel, factor, rows mask)]."""
    x = rng.standard_normal((R, G)).astype(np.float32)
    for c, f, mask in spikes:
        x[mask, c] = f * np.sign(x[mask, c] + 1e-3)
    return to_bf16_bits(x)


def test_two_alternating_channels_need_m2():
    """Two persistent channels of equal size, each the group maximum on about half the rows: one
    entry keeps the more frequent one; two entries keep both (each is an event on every row as a
    top-2 channel)."""
    R, G = 400, 32
    rng = np.random.default_rng(5)
    big = np.zeros(R, bool)
    big[::2] = True
    X = _group_rows(R, G, rng, [(3, 40.0, big), (17, 30.0, ~big), (3, 30.0, ~big), (17, 40.0, big)])
    L1, h1, e1 = oracle.build_table_multi(X, G, 1)
    assert L1[0, 0] in (3, 17) and e1[0] == R
    L2, h2, e2 = oracle.build_table_multi(X, G, 2)
    assert sorted(L2[0].tolist()) == [3, 17]
    assert h2[0].tolist() == [R, R]
    L3, h3, _ = oracle.build_table_multi(X, G, 3)
    assert sorted(L3[0, :2].tolist()) == [3, 17] and L3[0, 2] == -1  # no third consistent channel


def test_dominant_and_weaker_persistent_channel():
    """A dominant channel (60) and a weaker persistent one (20, above alpha * mean = 5 * ~3.25 on
    every row): m=1 finds only the dominant one, m=2 adds the weaker as its second entry; a
    weak channel of 12 stays below the event threshold and is not kept."""
    R, G = 300, 32
    rng = np.random.default_rng(6)
    allr = np.ones(R, bool)
    X = _group_rows(R, G, rng, [(9, 60.0, allr), (22, 20.0, allr)])
    L1, _, _ = oracle.build_table_multi(X, G, 1)
    assert L1[0].tolist() == [9]
    L2, h2, _ = oracle.build_table_multi(X, G, 2)
    assert L2[0].tolist() == [9, 22] and h2[0].tolist() == [R, R]
    X = _group_rows(R, G, np.random.default_rng(6), [(9, 60.0, allr), (22, 12.0, allr)])
    L2, h2, _ = oracle.build_table_multi(X, G, 2)
    assert L2[0].tolist() == [9, -1]


def test_rho_boundary_and_no_events():
    R, G = 200, 32
    rng = np.random.default_rng(8)
    rows = np.zeros(R, bool)
    rows[:70] = True  # channel 5 persistent on exactly 35 % of the rows
    X = _group_rows(R, G, rng, [(5, 50.0, rows)])
    L, h, e = oracle.build_table_multi(X, G, 2, rho=0.35)
    assert L[0, 0] == 5 and h[0, 0] == 70
    L, h, e = oracle.build_table_multi(X, G, 2, rho=0.36)
    assert L[0].tolist() == [-1, -1]
    quiet = to_bf16_bits(np.ones((R, G), np.float32))  # no row exceeds alpha * mean
    L, h, e = oracle.build_table_multi(quiet, G, 3)
    assert L[0].tolist() == [-1, -1, -1] and e[0] == 0


def test_multi_recovers_two_planted_channels():
    w = synth.two_outlier_groups(S=16)
    L, _, _ = oracle.build_table_multi(w.calib, w.G, 2)
    np.testing.assert_array_equal(np.sort(L, axis=1), np.sort(w.L, axis=1))
