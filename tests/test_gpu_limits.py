"""GPU parity at the limits the C ABI states: the largest table (K = OSC_MAX_GROUPS compensation
columns, one and two channels per group) and the largest row count (2^24 - 1 rows, where a
panel's byte offsets approach the 32-bit lane offsets of the GEMM's loads).  Same bar as the other
parity tests: quantized bytes bit-exact against the oracle, Y within 2e-3 * (|Y| + RMS(Y))."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from gpu_util import (DEV, assert_y_close, codes_rm, dev_bits16, gemm_multi, host_bits16, host_u8, host_y,  # noqa: E402
                      pack_multi, quant_multi, scales_rm, side_rm)


def table(rng, K, G, m):
    L = np.full((K, m), -1, np.int32)
    for k in range(K):
        L[k] = np.where(rng.random(m) < 0.8, rng.choice(G, size=m, replace=False), -1)
    return L


@pytest.mark.parametrize("H,G,m,S", [(16384, 16, 1, 40), (16384, 16, 1, 8), (8192, 16, 2, 40), (65536, 64, 1, 6)])
def test_largest_tables(H, G, m, S):
    K = H // G
    assert K * m == osc.OSC_MAX_GROUPS
    N = 96
    rng = np.random.default_rng(H + m + S)
    L = table(rng, K, G, m)
    X = synth.random_bf16((S, H), seed=S + m, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + m, scale=0.05)
    QX, SX, B = quant_multi(dev_bits16(X), S, H, G, L, m)
    QW, SW, WL = pack_multi(dev_bits16(W), N, H, G, L, m)
    Y = gemm_multi(QX, SX, B, QW, SW, WL, S, N, H, G, m)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act_multi(X, G, L, m)
    np.testing.assert_array_equal(codes_rm(QX, S, H, osc.OSC_MXFP4), rq)
    np.testing.assert_array_equal(scales_rm(SX, S, H, G), rs)
    np.testing.assert_array_equal(side_rm(B, S, H, G, m), rb)
    wq, ws, wl = oracle.pack_weights_multi(W, G, L, m)
    np.testing.assert_array_equal(codes_rm(QW, N, H, osc.OSC_MXFP4), wq)
    np.testing.assert_array_equal(side_rm(WL, N, H, G, m), wl)
    ref = oracle.gemm_comp(rq, rs, wq, ws, G, rb, wl)
    assert_y_close(host_y(Y), ref, what=f"K*m = {K * m}, S = {S}")


def test_most_rows():
    """2^24 - 1 rows (H=256, G=32): the quantized operands' panels hold 1 GiB of codes each and the
    last 256-row tile is ragged.  Inputs are drawn on the device from a seeded generator; the
    oracle checks sampled rows (including the last ones) of the codes, scales, B and Y."""
    R, H, G, N = (1 << 24) - 1, 256, 32, 128
    K = H // G
    gen = torch.Generator(device=DEV)
    gen.manual_seed(24)
    X = torch.randn((R, H), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    rng = np.random.default_rng(24)
    L = table(rng, K, G, 1)
    W = synth.random_bf16((N, H), seed=25, scale=0.05)
    QX, SX, B = quant_multi(X, R, H, G, L, 1)
    QW, SW, WL = pack_multi(dev_bits16(W), N, H, G, L, 1)
    Y = gemm_multi(QX, SX, B, QW, SW, WL, R, N, H, G, 1)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(R, 40, replace=False), np.arange(R - 300, R), np.arange(0, 4)]))
    ridx = torch.from_numpy(rows).to(DEV)
    Xs = host_bits16(X.index_select(0, ridx))
    # the tiled buffers, restricted to the sampled rows (a permutation, undone on the host)
    codes = QX.view(H // 128, R, 64).index_select(1, ridx).cpu().numpy().transpose(1, 0, 2).reshape(len(rows), H // 2)
    scl = SX.view(K // 4, R, 4).index_select(1, ridx).cpu().numpy().transpose(1, 0, 2).reshape(len(rows), K)
    side = B.view(1, R, 32).index_select(1, ridx).cpu().view(torch.int16).numpy().view(np.uint16)
    side = side.transpose(1, 0, 2).reshape(len(rows), 32)[:, :K]
    rq, rs, rb = oracle.quant_act_multi(Xs, G, L, 1)
    np.testing.assert_array_equal(codes, rq)
    np.testing.assert_array_equal(scl, rs)
    np.testing.assert_array_equal(side, rb)
    ref = oracle.osc_linear_multi(Xs, W, G, L, 1)
    assert_y_close(Y.index_select(0, ridx).double().cpu().numpy(), ref, what="2^24 - 1 rows")
    del X, QX, SX, B, Y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("R", [2796202, 2796203])
def test_fp6p_descriptor_limit(R):
    """E3M2 pairs at H=1024 (eight 128-channel panels of R x 96 bytes of codes): the pair GEMM's main
    loop reads each operand region through one descriptor with 32-bit offsets while the codes are
    under 2 GiB.  2796202 rows end the last panel 512 bytes under 2^31 (that loop, at its largest
    offsets); 2796203 rows pass 2^31 and take the general stage path.  Inputs are drawn on the device
    from a seeded generator; the oracle checks sampled rows (including the last ones) of the codes,
    scales, B and Y."""
    H, G, N, m = 1024, 16, 128, 1
    K, P = H // G, H // 128
    assert (P * R * 96 < 1 << 31) == (R == 2796202)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(R % 1000)
    X = torch.randn((R, H), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    rng = np.random.default_rng(R % 1000)
    L = table(rng, K, G, m)
    W = synth.random_bf16((N, H), seed=26, scale=0.05)
    QX, SX, B = quant_multi(X, R, H, G, L, m, osc.OSC_FP6P)
    QW, SW, WL = pack_multi(dev_bits16(W), N, H, G, L, m, osc.OSC_FP6P)
    Y = torch.empty((R, N), dtype=torch.float32, device=DEV)
    osc.osc_gemm_fp6p(QX, SX, B, QW, SW, WL, R, N, H, m, Y, osc.OSC_Y_F32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.choice(R, 40, replace=False), np.arange(R - 300, R), np.arange(0, 4)]))
    ridx = torch.from_numpy(rows).to(DEV)
    Xs = host_bits16(X.index_select(0, ridx))
    # the tiled pair codes restricted to the sampled rows: per 128-channel panel the R x 64 first
    # region, then the R x 32 second region with block b's 8 bytes at 8 * (b ^ (((r >> 1) ^ (r >> 3)) & 3))
    q = QX.view(P, R * 96)
    first = q[:, :R * 64].reshape(P, R, 4, 16).index_select(1, ridx).cpu().numpy()
    second = q[:, R * 64:].reshape(P, R, 4, 8).index_select(1, ridx).cpu().numpy()
    r = rows[:, None]
    pos = np.arange(4)[None, :] ^ (((r >> 1) ^ (r >> 3)) & 3)
    second = second[:, np.arange(len(rows))[:, None], pos, :]
    codes = np.concatenate([first, second], axis=3).transpose(1, 0, 2, 3).reshape(len(rows), P * 96)
    scl = SX.view(P, R, 4).index_select(1, ridx).cpu().numpy().transpose(1, 0, 2).reshape(len(rows), H // 32)
    npn = (K * m + 31) // 32
    side = B.view(npn, R, 32).index_select(1, ridx).cpu().view(torch.int16).numpy().view(np.uint16)
    side = side.transpose(1, 0, 2).reshape(len(rows), npn * 32)[:, :K * m]
    rq, rs, rb = oracle.quant_act_fp6p(Xs, L, m)
    np.testing.assert_array_equal(codes, rq)
    np.testing.assert_array_equal(scl, rs)
    np.testing.assert_array_equal(side, rb)
    rqw, rsw, rwl = oracle.pack_weights_fp6p(W, L, m)
    ref = oracle.gemm_fp6p(rq, rs, rqw, rsw, rb, rwl)
    assert_y_close(Y.index_select(0, ridx).double().cpu().numpy(), ref, what=f"E3M2 pairs, {R} rows")
    del X, QX, SX, B, Y
    torch.cuda.empty_cache()
