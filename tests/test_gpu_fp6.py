"""GPU parity of the E3M2-pair path for G = 16 (osc_quant_act_multi / osc_pack_weights_multi with
OSC_FP6P, osc_gemm_fp6p) against the oracle's pair re-encoding (tests/test_oracle_fp6.py pins it
to the G = 16 MXFP4 oracle).  Codes, scales and B bit-exact -- including pairs whose scale codes
differ by up to 9, where the smaller group rounds -- and Y within 2e-3 * (|Y| + RMS(Y))."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import to_bf16_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from gpu_util import (assert_y_close, codes6_rm, dev_bits16, gemm_fp6p, gemm_multi, host_y, pack_multi,  # noqa: E402
                      quant_multi, scales_rm, side_rm)

FP6P = osc.OSC_FP6P


def crafted_rows(rng, S, H):
    """Every 32-channel pair gets a larger group with amax 2^a and a smaller one 2^(a - gap),
    gap 0..9, values spread over every E2M1 magnitude of both groups, random signs."""
    x = np.zeros((S, H))
    mags = np.array([0.0, 0.3, 0.5, 0.8, 1.0, 1.25, 1.5, 2.0, 2.6, 3.0, 3.6, 4.0, 5.0, 6.0, 0.1, 0.2])
    for s in range(S):
        for b in range(H // 32):
            a = int(rng.integers(-8, 8))
            gap = int(rng.integers(0, 10))
            big, small = (0, 1) if rng.random() < 0.5 else (1, 0)
            for g, e in ((big, a), (small, a - gap)):
                v = rng.permutation(mags) * 2.0 ** (e - 2)
                v[0] = 6.0 * 2.0 ** (e - 2) * 1.2  # the group's amax lands in [4, 8) * 2^(e - 2)
                x[s, 32 * b + 16 * g:32 * b + 16 * g + 16] = v * rng.choice([-1.0, 1.0], 16)
    return to_bf16_bits(x)


@pytest.mark.parametrize("m", [0, 1, 2])
@pytest.mark.parametrize("data", ["random", "crafted"])
def test_quant_fp6p_bit_exact(m, data):
    S, H = 37, 1024
    rng = np.random.default_rng(10 * m + (data == "crafted"))
    X = synth.random_bf16((S, H), seed=m + 1, scale=2.0) if data == "random" else crafted_rows(rng, S, H)
    L = None
    if m:
        L = np.full((H // 16, m), -1, np.int32)
        for k in range(H // 16):
            L[k] = rng.choice(16, size=m, replace=False)
    QX, SX, B = quant_multi(dev_bits16(X), S, H, 16, L, max(m, 1), FP6P) if m else \
        _quant_plain(dev_bits16(X), S, H)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act_fp6p(X, L, max(m, 1))
    np.testing.assert_array_equal(codes6_rm(QX, S, H), rq)
    np.testing.assert_array_equal(scales_rm(SX, S, H, 32), rs)
    if m:
        np.testing.assert_array_equal(side_rm(B, S, H, 16, m), rb)


def test_quant_fp6p_exhaustive_bf16():
    """Every finite bf16 pattern (subnormals, zeros of both signs, the largest magnitudes), sorted,
    reversed and shuffled, so that pairs meet scale-code gaps from 0 to over 200; one protected
    channel per 16-group."""
    from synth import bits_to_f32
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = np.where(np.isfinite(bits_to_f32(bits)), bits, 0).astype(np.uint16)
    rng = np.random.default_rng(16)
    X = np.stack([bits, bits[::-1].copy()] + [rng.permutation(bits) for _ in range(4)]).reshape(-1, 8192)
    S, H = X.shape
    L = rng.integers(-1, 16, (H // 16, 1)).astype(np.int32)
    QX, SX, B = quant_multi(dev_bits16(X), S, H, 16, L, 1, FP6P)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act_fp6p(X, L, 1)
    np.testing.assert_array_equal(scales_rm(SX, S, H, 32), rs)
    np.testing.assert_array_equal(codes6_rm(QX, S, H), rq)
    np.testing.assert_array_equal(side_rm(B, S, H, 16, 1), rb)


def _quant_plain(Xd, S, H):
    from gpu_util import _tiled_outputs
    QX, SX, _ = _tiled_outputs(S, H, 16, FP6P, False)
    osc.osc_quant_act(Xd, S, H, 16, None, FP6P, QX, SX, None)
    return QX, SX, None


def test_pack_weights_fp6p_bit_exact():
    N, H = 100, 512
    W = synth.random_bf16((N, H), seed=9, scale=0.05)
    L = np.random.default_rng(9).integers(-1, 16, (H // 16, 1)).astype(np.int32)
    QW, SW, WL = pack_multi(dev_bits16(W), N, H, 16, L, 1, FP6P)
    torch.cuda.synchronize()
    rq, rs, rwl = oracle.pack_weights_fp6p(W, L, 1)
    np.testing.assert_array_equal(codes6_rm(QW, N, H), rq)
    np.testing.assert_array_equal(scales_rm(SW, N, H, 32), rs)
    np.testing.assert_array_equal(side_rm(WL, N, H, 16, 1), rwl)


@pytest.mark.parametrize("S,N,H,m", [(40, 96, 512, 1), (8, 64, 256, 2), (300, 520, 768, 1), (77, 200, 1024, 0),
                                     (600, 1536, 512, 3)])
def test_gemm_fp6p(S, N, H, m):
    rng = np.random.default_rng(S + N + H + m)
    X = synth.random_bf16((S, H), seed=S, scale=2.0)
    W = synth.random_bf16((N, H), seed=N, scale=0.05)
    L = None
    if m:
        L = np.full((H // 16, m), -1, np.int32)
        for k in range(H // 16):
            L[k] = rng.choice(16, size=m, replace=False)
    mm = max(m, 1)
    if m:
        QX, SX, B = quant_multi(dev_bits16(X), S, H, 16, L, mm, FP6P)
        QW, SW, WL = pack_multi(dev_bits16(W), N, H, 16, L, mm, FP6P)
    else:
        QX, SX, B = _quant_plain(dev_bits16(X), S, H)
        from gpu_util import _tiled_outputs
        QW, SW, WL = _tiled_outputs(N, H, 16, FP6P, False)
        osc.osc_pack_weights(dev_bits16(W), N, H, 16, None, FP6P, QW, SW, None)
    Y = gemm_fp6p(QX, SX, B, QW, SW, WL, S, N, H, mm)
    torch.cuda.synchronize()
    rqx, rsx, rb = oracle.quant_act_fp6p(X, L, mm)
    rqw, rsw, rwl = oracle.pack_weights_fp6p(W, L, mm)
    ref = oracle.gemm_fp6p(rqx, rsx, rqw, rsw, rb, rwl)
    assert_y_close(host_y(Y), ref, what=f"fp6p S={S} N={N} H={H} m={m}")
    # the same layer at G = 16 in MXFP4 (every pair exact on these inputs): same Y within tolerance
    if m:
        QX4, SX4, B4 = quant_multi(dev_bits16(X), S, H, 16, L, mm)
        QW4, SW4, WL4 = pack_multi(dev_bits16(W), N, H, 16, L, mm)
        Y4 = gemm_multi(QX4, SX4, B4, QW4, SW4, WL4, S, N, H, 16, mm)
        torch.cuda.synchronize()
        assert_y_close(host_y(Y), host_y(Y4), what="fp6p against the MXFP4 G=16 path")


def test_gemm_fp6p_sweep_workload():
    """The G-sweep workload at G = 16 (S = 8192, H = 4096, N = 6144, its table): sampled rows and
    columns against the oracle, in the configuration the benchmark times."""
    w = synth.group_sweep(8192, 16)
    L, _, _ = oracle.build_table(w.calib, 16)
    L2 = L.reshape(-1, 1)
    QX, SX, B = quant_multi(dev_bits16(w.X), w.S, w.H, 16, L2, 1, FP6P)
    QW, SW, WL = pack_multi(dev_bits16(w.W), w.N, w.H, 16, L2, 1, FP6P)
    Y = gemm_fp6p(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, 1)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(2).choice(w.S, 16, replace=False))
    cols = np.sort(np.random.default_rng(3).choice(w.N, 512, replace=False))
    rqx, rsx, rb = oracle.quant_act_fp6p(w.X[rows], L, 1)
    rqw, rsw, rwl = oracle.pack_weights_fp6p(w.W[cols], L, 1)
    ref = oracle.gemm_fp6p(rqx, rsx, rqw, rsw, rb, rwl)
    got = Y.index_select(0, torch.from_numpy(rows).to(Y.device)).index_select(1, torch.from_numpy(cols).to(Y.device))
    assert_y_close(got.double().cpu().numpy(), ref, what="fp6p G-sweep S=8192")


def _e2m1_values(Q4, H):
    """uint8[R, H/2] MXFP4 codes (channel 2i in the low nibble of byte i) -> float64[R, H] E2M1 values."""
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    c = np.empty((Q4.shape[0], H), np.uint8)
    c[:, 0::2] = Q4 & 15
    c[:, 1::2] = Q4 >> 4
    return np.where(c & 8, -1.0, 1.0) * mag[c & 7]


def _e3m2_values(Q6, H):
    """uint8[R, 3H/4] packed E3M2 codes -> float64[R, H] values (sign bit 5, exponent bits 4..2 with
    bias 3, mantissa bits 1..0; exponent 0: multiples of 1/16)."""
    out = np.empty((Q6.shape[0], H))
    for k in range(H):
        c = oracle.get_code6(Q6, k).astype(np.int64)
        e, m = (c >> 2) & 7, c & 3
        mag = np.where(e == 0, m / 16.0, (1.0 + m / 4.0) * np.exp2(e - 3.0))
        out[:, k] = np.where(c & 32, -mag, mag)
    return out


def test_fp6p_changes_only_pairs_more_than_5_scale_codes_apart():
    """Against the exact G = 16 MXFP4 quantization (the oracle at G = 16): the GPU's E3M2 pairs carry
    every element exactly in pairs whose two scale codes differ by at most 5, and the larger group of
    every pair exactly; in pairs further apart the smaller group's elements move by at most half an
    E3M2 step (1/32 of the pair scale), and on these rows (gaps up to 9) some do move.  Y of the pair
    GEMM differs from Y of the exact G = 16 layer by no more than those moves can make it."""
    S, H, N = 48, 1024, 96
    rng = np.random.default_rng(77)
    X = crafted_rows(rng, S, H)
    W = synth.random_bf16((N, H), seed=78, scale=0.05)
    QX, SX, _ = _quant_plain(dev_bits16(X), S, H)
    from gpu_util import _tiled_outputs
    QW, SW, _ = _tiled_outputs(N, H, 16, FP6P, False)
    osc.osc_pack_weights(dev_bits16(W), N, H, 16, None, FP6P, QW, SW, None)
    Y = gemm_fp6p(QX, SX, None, QW, SW, None, S, N, H, 1)
    torch.cuda.synchronize()

    def pair_values(Q6, S32, R):
        return _e3m2_values(Q6, H) * np.exp2(np.repeat(S32.astype(np.float64) - 127.0, 32, axis=1))

    def exact_values(A, R):
        q4, s16, _ = oracle.quant_act(A, 16, None)
        return _e2m1_values(q4, H) * np.exp2(np.repeat(s16.astype(np.float64) - 127.0, 16, axis=1)), s16

    got_x = pair_values(codes6_rm(QX, S, H), scales_rm(SX, S, H, 32), S)
    ex_x, s16 = exact_values(X, S)
    s = s16.astype(int)
    gap = np.abs(s[:, 0::2] - s[:, 1::2])                                   # [S, H/32]
    small = np.where(s[:, 0::2] < s[:, 1::2], 0, 1)                         # which 16-group is smaller
    E = np.maximum(np.maximum(s[:, 0::2], s[:, 1::2]) - 2, 0)
    d = got_x - ex_x
    for b in range(H // 32):
        blk = slice(32 * b, 32 * b + 32)
        near = gap[:, b] <= 5
        assert np.all(d[near, blk] == 0.0), f"pair {b}: a pair within 5 scale codes changed"
        for g in (0, 1):
            grp = slice(32 * b + 16 * g, 32 * b + 16 * g + 16)
            bigger = ~near & (small[:, b] != g)
            assert np.all(d[bigger, grp] == 0.0), f"pair {b}: the larger group changed"
            smaller = ~near & (small[:, b] == g)
            half_step = np.exp2(E[smaller, b] - 127.0 - 5.0)[:, None]
            assert np.all(np.abs(d[smaller, grp]) <= half_step), f"pair {b}: moved by more than half a step"
    assert np.count_nonzero(d) > 0 and np.all(gap.max() > 5)

    got_w = pair_values(*[codes6_rm(QW, N, H), scales_rm(SW, N, H, 32)], N)
    ex_w, _ = exact_values(W, N)
    dw = got_w - ex_w
    y_exact = ex_x @ ex_w.T
    bound = np.abs(d) @ np.abs(ex_w).T + np.abs(ex_x) @ np.abs(dw).T + np.abs(d) @ np.abs(dw).T
    y = host_y(Y).astype(np.float64)
    # fp32 accumulation on top of the bound: 2e-6 of the sum of magnitudes
    slack = 2e-6 * (np.abs(got_x) @ np.abs(got_w).T)
    assert np.all(np.abs(y - y_exact) <= bound + slack)
    assert np.any(np.abs(y - y_exact) > slack)  # the moves do reach Y on these rows
