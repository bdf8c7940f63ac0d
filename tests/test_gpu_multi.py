"""GPU parity of the several-channels-per-group calls (osc_*_multi; the outlook section's 2-3
channel direction of the OSC page) against the oracle's *_multi functions, through the C ABI.
Bar as for the single-channel path: codes, scales, B and W_L bit-exact, the table exact, Y within
|dY| <= 2e-3 * (|Y| + RMS(Y)); m = 1 must reproduce the single-channel calls bit for bit."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from gpu_util import (assert_y_close, codes_rm, dev_bits16, gemm, gemm_multi, host_y, pack, pack_multi,  # noqa: E402
                      quant, quant_multi, scales_rm, side_rm)


@functools.lru_cache(maxsize=None)
def two():
    return synth.two_outlier_groups(S=2048)


def random_multi_table(rng, K, G, m, p_none=0.25):
    L = np.full((K, m), -1, np.int32)
    for k in range(K):
        ch = rng.choice(G, size=m, replace=False)
        L[k] = np.where(rng.random(m) >= p_none, ch, -1)
    return L


@pytest.mark.parametrize("G,m", [(16, 3), (32, 2), (32, 3), (64, 2)])
def test_quant_multi_bit_exact(G, m):
    S, H = 77, 1024
    X = synth.random_bf16((S, H), seed=G + m, scale=3.0)
    L = random_multi_table(np.random.default_rng(G * m), H // G, G, m)
    QX, SX, B = quant_multi(dev_bits16(X), S, H, G, L, m)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act_multi(X, G, L, m)
    np.testing.assert_array_equal(codes_rm(QX, S, H, osc.OSC_MXFP4), rq)
    np.testing.assert_array_equal(scales_rm(SX, S, H, G), rs)
    np.testing.assert_array_equal(side_rm(B, S, H, G, m), rb)


@pytest.mark.parametrize("G,m", [(16, 2), (16, 3), (32, 2), (64, 3)])
def test_quant_multi_entries_sharing_a_dword(G, m):
    """Entries on the two channels of one 32-bit word of X (2j and 2j+1, listed in either order),
    and for G = 64 entries in both halves of the group: each listed slot is zeroed and copied."""
    S, H = 40, 1024
    X = synth.random_bf16((S, H), seed=G + 10 * m, scale=3.0)
    rng = np.random.default_rng(G + m)
    K = H // G
    L = np.full((K, m), -1, np.int32)
    for k in range(K):
        j = 2 * int(rng.integers(0, G // 2))
        pair = [j, j + 1] if k % 2 else [j + 1, j]
        rest = [c for c in rng.permutation(G) if c not in pair]
        if G == 64:  # the third entry in the other half
            rest = [c for c in rest if (c >= 32) != (j >= 32)]
        L[k] = (pair + rest)[:m]
    QX, SX, B = quant_multi(dev_bits16(X), S, H, G, L, m)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act_multi(X, G, L, m)
    np.testing.assert_array_equal(codes_rm(QX, S, H, osc.OSC_MXFP4), rq)
    np.testing.assert_array_equal(scales_rm(SX, S, H, G), rs)
    np.testing.assert_array_equal(side_rm(B, S, H, G, m), rb)


def test_quant_and_pack_two_outlier_workload():
    w = two()
    QX, SX, B = quant_multi(dev_bits16(w.X), w.S, w.H, w.G, w.L, 2)
    QW, SW, WL = pack_multi(dev_bits16(w.W), w.N, w.H, w.G, w.L, 2)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act_multi(w.X, w.G, w.L, 2)
    np.testing.assert_array_equal(codes_rm(QX, w.S, w.H, osc.OSC_MXFP4), rq)
    np.testing.assert_array_equal(scales_rm(SX, w.S, w.H, w.G), rs)
    np.testing.assert_array_equal(side_rm(B, w.S, w.H, w.G, 2), rb)
    rows = np.sort(np.random.default_rng(3).choice(w.N, 512, replace=False))
    wq, ws, wl = oracle.pack_weights_multi(w.W[rows], w.G, w.L, 2)
    np.testing.assert_array_equal(codes_rm(QW, w.N, w.H, osc.OSC_MXFP4)[rows], wq)
    np.testing.assert_array_equal(scales_rm(SW, w.N, w.H, w.G)[rows], ws)
    np.testing.assert_array_equal(side_rm(WL, w.N, w.H, w.G, 2)[rows], wl)


def test_gemm_multi_two_outlier_sampled():
    w = two()
    QX, SX, B = quant_multi(dev_bits16(w.X), w.S, w.H, w.G, w.L, 2)
    QW, SW, WL = pack_multi(dev_bits16(w.W), w.N, w.H, w.G, w.L, 2)
    Y = gemm_multi(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G, 2)
    torch.cuda.synchronize()
    got = host_y(Y)
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(w.S, 24, replace=False))
    cols = np.sort(rng.choice(w.N, 2048, replace=False))
    rq, rs, rb = oracle.quant_act_multi(w.X[rows], w.G, w.L, 2)
    wq, ws, wl = oracle.pack_weights_multi(w.W[cols], w.G, w.L, 2)
    assert_y_close(got[np.ix_(rows, cols)], oracle.gemm_comp(rq, rs, wq, ws, w.G, rb, wl), what="two-outlier m=2")


@pytest.mark.parametrize("S,N,H,G,m", [(77, 200, 512, 32, 3), (130, 72, 512, 16, 2), (33, 300, 1024, 64, 2),
                                       (5, 64, 256, 32, 2)])
def test_gemm_multi_ragged(S, N, H, G, m):
    X = synth.random_bf16((S, H), seed=S + m, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + m, scale=0.05)
    L = random_multi_table(np.random.default_rng(H + G + m), H // G, G, m)
    QX, SX, B = quant_multi(dev_bits16(X), S, H, G, L, m)
    QW, SW, WL = pack_multi(dev_bits16(W), N, H, G, L, m)
    Y = gemm_multi(QX, SX, B, QW, SW, WL, S, N, H, G, m)
    torch.cuda.synchronize()
    assert_y_close(host_y(Y), oracle.osc_linear_multi(X, W, G, L, m), what=f"{S}x{N}x{H} G={G} m={m}")


def test_m1_multi_calls_equal_single_calls():
    w = synth.tiny()
    Xd, Wd = dev_bits16(w.X), dev_bits16(w.W)
    a = quant(Xd, w.S, w.H, w.G, w.L, osc.OSC_MXFP4)
    b = quant_multi(Xd, w.S, w.H, w.G, w.L.reshape(-1, 1), 1)
    pa = pack(Wd, w.N, w.H, w.G, w.L, osc.OSC_MXFP4)
    pb = pack_multi(Wd, w.N, w.H, w.G, w.L.reshape(-1, 1), 1)
    Ya = gemm(*a, *pa, w.S, w.N, w.H, w.G)
    Yb = gemm_multi(*b, *pb, w.S, w.N, w.H, w.G, 1)
    torch.cuda.synchronize()
    for x, y in zip(a + pa, b + pb):
        assert torch.equal(x, y)
    assert torch.equal(Ya, Yb)


@pytest.mark.parametrize("name,m", [("two", 2), ("two", 3), ("qkv", 3)])
def test_build_table_multi(name, m):
    w = two() if name == "two" else synth.qkv(S=16)
    K = w.H // w.G
    L = torch.full((K * m,), -7, dtype=torch.int32, device="cuda:0")
    hits = torch.full((K * m,), -7, dtype=torch.int32, device="cuda:0")
    ev = torch.full((K,), -7, dtype=torch.int32, device="cuda:0")
    osc.osc_build_table_multi(dev_bits16(w.calib), w.calib.shape[0], w.H, w.G, 5.0, 0.35, m, L, hits, ev)
    torch.cuda.synchronize()
    rL, rh, re = oracle.build_table_multi(w.calib, w.G, m)
    np.testing.assert_array_equal(L.cpu().numpy().reshape(K, m), rL)
    np.testing.assert_array_equal(hits.cpu().numpy().reshape(K, m), rh)
    np.testing.assert_array_equal(ev.cpu().numpy(), re)
