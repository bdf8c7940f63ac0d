"""GPU parity at the shapes and kernel configurations the benchmark times beyond the headline:
the FP8-activation prefill GEMM at G = 64 (the down-projection W2 of the block, where the
group-size rule picks G = 64), the forced-OSC W2 at its own shape, the attention output
projection Wo, and the block's gated MLP at S = 4096 through the executor, stage by stage.

Bar as everywhere: codes and scales bit-exact (sampled rows), Y within |dY| <= 2e-3 (|Y| + RMS(Y))
on sampled rows x 2048 columns and on every row x 24 columns, fp32 output.  The oracle follows the
OSC page §3.2 (dual path), §4 (FP8 fallback) and §6 (group size)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import bits_to_f32

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from w4a4_outlier_split_amd import block as blk  # noqa: E402
from gpu_util import (DEV, assert_y_close, codes_rm, dev_bits16, gemm, gemm_fp8, host_bits16, host_y, pack,  # noqa: E402
                      quant, scales_rm, side_rm)

FP4, FP8 = osc.OSC_MXFP4, osc.OSC_MXFP8


def sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    idx.update({0, n - 1})
    return np.array(sorted(idx))


def check_sampled(got, X, W, G, L, afmt, wfmt, seed, what):
    """got [S, N] device output (host fp64); the oracle on sampled rows x 2048 columns and on every
    row x 24 columns.  L is None on the FP8 path."""
    S, N = got.shape
    rows, wide, cols = sample(S, 24, seed), sample(N, 2048, seed + 1), sample(N, 24, seed + 2)
    rq, rs, rb = oracle.quant_act(X[rows], G, L, afmt)
    wq, ws, wl = oracle.pack_weights(W[wide], G, L, wfmt)
    ref_rows = oracle.gemm(rq, rs, wq, ws, G, rb, wl, afmt=afmt, wfmt=wfmt)
    xq, xs, xb = oracle.quant_act(X, G, L, afmt)
    cq, cs, cl = oracle.pack_weights(W[cols], G, L, wfmt)
    ref_cols = oracle.gemm(xq, xs, cq, cs, G, xb, cl, afmt=afmt, wfmt=wfmt)
    rms = float(np.sqrt(np.mean(ref_rows ** 2)))
    assert_y_close(got[np.ix_(rows, wide)], ref_rows, rms, what=f"{what} rows")
    assert_y_close(got[:, cols], ref_cols, rms, what=f"{what} cols")


@pytest.mark.parametrize("wfmt", [FP4, FP8])
def test_gemm_fp8_g64_down_proj_shape(wfmt):
    """W2 of the block: S=4096, H=12288, N=4096, FP8 activations at G = 64 on the prefill kernel
    (256x256 tiles, the G = 64 scale half-stages)."""
    w = synth.ffn_down(S=4096)
    G = 64
    QX, SX, _ = quant(dev_bits16(w.X), w.S, w.H, G, None, FP8)
    QW, SW, _ = pack(dev_bits16(w.W), w.N, w.H, G, None, wfmt)
    Y = gemm_fp8(QX, SX, QW, SW, wfmt, w.S, w.N, w.H, G)
    torch.cuda.synchronize()
    rows = sample(w.S, 64, 11)
    rq, rs, _ = oracle.quant_act(w.X[rows], G, None, FP8)
    np.testing.assert_array_equal(codes_rm(QX, w.S, w.H, FP8)[rows], rq)
    np.testing.assert_array_equal(scales_rm(SX, w.S, w.H, G)[rows], rs)
    check_sampled(host_y(Y), w.X, w.W, G, None, FP8, wfmt, 12, f"W2 FP8 G=64 wfmt={wfmt}")


@pytest.mark.parametrize("S,N,H,wfmt", [(77, 200, 512, FP8), (77, 136, 768, FP4), (300, 264, 1280, FP8)])
def test_gemm_fp8_g64_ragged(S, N, H, wfmt):
    """G = 64 FP8 activations with more rows than the decode kernel takes: ragged S and N."""
    G = 64
    X = synth.random_bf16((S, H), seed=S + 1, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + 2, scale=0.05)
    QX, SX, _ = quant(dev_bits16(X), S, H, G, None, FP8)
    QW, SW, _ = pack(dev_bits16(W), N, H, G, None, wfmt)
    Y = gemm_fp8(QX, SX, QW, SW, wfmt, S, N, H, G)
    torch.cuda.synchronize()
    rq, rs, _ = oracle.quant_act(X, G, None, FP8)
    wq, ws, _ = oracle.pack_weights(W, G, None, wfmt)
    assert_y_close(host_y(Y), oracle.gemm(rq, rs, wq, ws, G, afmt=FP8, wfmt=wfmt), what=f"fp8 G=64 {S}x{N}x{H}")


def osc_layer(w, L):
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G)
    torch.cuda.synchronize()
    return QX, SX, B, Y


def test_forced_osc_down_proj_shape():
    """W2 on the 4-bit OSC path at its own shape (S=4096, H=12288, N=4096, K=384 compensation
    columns, 256x256 tiles), the table built by the oracle from the calibration rows."""
    w = synth.ffn_down(S=4096)
    L, _, _ = oracle.build_table(w.calib, w.G)
    assert (L >= 0).sum() == 96
    QX, SX, B, Y = osc_layer(w, L)
    rows = sample(w.S, 64, 21)
    rq, rs, rb = oracle.quant_act(w.X[rows], w.G, L, FP4)
    np.testing.assert_array_equal(codes_rm(QX, w.S, w.H, FP4)[rows], rq)
    np.testing.assert_array_equal(scales_rm(SX, w.S, w.H, w.G)[rows], rs)
    np.testing.assert_array_equal(side_rm(B, w.S, w.H, w.G)[rows], rb)
    check_sampled(host_y(Y), w.X, w.W, w.G, L, FP4, FP4, 22, "forced-OSC W2")


def test_attn_out_proj_shape():
    """Wo of the block: S=4096, H=N=4096, G=32, table from the oracle."""
    w = synth.attn_out(S=4096)
    L, _, _ = oracle.build_table(w.calib, w.G)
    QX, SX, B, Y = osc_layer(w, L)
    check_sampled(host_y(Y), w.X, w.W, w.G, L, FP4, FP4, 31, "Wo")


def dev_bf16(a):
    return dev_bits16(a).view(torch.bfloat16)


def test_block_mlp_s4096_stage_by_stage():
    """The block's gated MLP as the benchmark runs it: the FFN-up workload (S=4096, H=4096) through
    the stacked W1|W3 up-projection (N=24576) on the path and group size the rules pick, the glue
    fused into W2's input quantization, W2 (12288 -> 4096) on the rules' path (FP8 activations at
    G = 64 on these inputs).  Each stage is checked against the oracle fed with the device's
    previous output."""
    H, F = 4096, 12288
    wu = synth.ffn_up(S=4096)
    S = wu.S
    W2 = synth.draw_w(H, F, 35)
    cal_up = dev_bf16(wu.calib)
    g_up, _ = blk.calibrate_group_size(torch, cal_up, H)
    c_up = blk.calibrate(torch, cal_up, H, g_up)
    assert c_up.path == "osc"
    up = blk.Linear(torch, dev_bf16(wu.W), 2 * F, H, g_up, "osc", c_up.L)
    hc = blk.MLP(up, blk.Linear(torch, dev_bf16(W2), H, F, 32, "fp8")).glue_rows(torch, cal_up)
    g_dn, _ = blk.calibrate_group_size(torch, hc, F)
    c_dn = blk.calibrate(torch, hc, F, g_dn)
    if c_dn.path == "fp8" and g_dn == 16:  # the FP8 path's scales cover 32 or 64 channels
        g_dn = 32
        c_dn = blk.calibrate(torch, hc, F, 32)
    del hc
    down = blk.Linear(torch, dev_bf16(W2), H, F, g_dn, c_dn.path, c_dn.L)
    mlp = blk.MLP(up, down)
    bufs = mlp.buffers(S, DEV)
    Y = torch.empty((S, H), dtype=torch.float32, device=DEV)
    mlp.forward(dev_bf16(wu.X), S, bufs, Y, osc.OSC_Y_F32)
    torch.cuda.synchronize()
    # stage 1: the up-projection (bf16 output: the tolerance plus its own rounding)
    GU = host_bits16(bufs["gu"].view(torch.int16))
    Lup = c_up.L[:, 0]
    rows, wide = sample(S, 16, 41), sample(2 * F, 2048, 42)
    rq, rs, rb = oracle.quant_act(wu.X[rows], g_up, Lup, FP4)
    wq, ws, wl = oracle.pack_weights(wu.W[wide], g_up, Lup, FP4)
    y1 = oracle.gemm(rq, rs, wq, ws, g_up, rb, wl)
    got1 = bits_to_f32(GU[np.ix_(rows, wide)]).astype(np.float64)
    rel = np.abs(got1 - y1) / (np.abs(y1) + np.sqrt(np.mean(y1 ** 2)))
    assert rel.max() <= 2e-3 + 2 ** -8, f"up-projection: max scaled error {rel.max():.3g}"
    # stage 2: glue + quantization of W2's input, bit for bit on the device's GU (sampled rows)
    afmt = FP4 if c_dn.path == "osc" else FP8
    L2 = c_dn.L[:, 0] if c_dn.path == "osc" else None
    QX, SX, B = bufs["h"]
    qrows = sample(S, 64, 43)
    hq, hs, hb = oracle.swiglu_quant(GU[qrows], g_dn, None if L2 is None else L2.reshape(-1, 1), 1, afmt)
    np.testing.assert_array_equal(codes_rm(QX, S, F, afmt)[qrows], hq)
    np.testing.assert_array_equal(scales_rm(SX, S, F, g_dn)[qrows], hs)
    if L2 is not None:
        np.testing.assert_array_equal(side_rm(B, S, F, g_dn)[qrows], hb)
    # stage 3: W2 on the device's own glue output, sampled rows x 2048 columns and all rows x 24
    aq, as_, ab = oracle.swiglu_quant(GU, g_dn, None if L2 is None else L2.reshape(-1, 1), 1, afmt)
    got = host_y(Y)
    r3, w3, c3 = sample(S, 24, 44), sample(H, 2048, 45), sample(H, 24, 46)
    qw, sw, wlw = oracle.pack_weights(W2[w3], g_dn, L2, FP4)
    ref_rows = oracle.gemm(aq[r3], as_[r3], qw, sw, g_dn, None if ab is None else ab[r3], wlw, afmt=afmt,
                           wfmt=FP4)
    cw, cs2, cl = oracle.pack_weights(W2[c3], g_dn, L2, FP4)
    ref_cols = oracle.gemm(aq, as_, cw, cs2, g_dn, ab, cl, afmt=afmt, wfmt=FP4)
    rms = float(np.sqrt(np.mean(ref_rows ** 2)))
    assert_y_close(got[np.ix_(r3, w3)], ref_rows, rms, what=f"W2 ({c_dn.path}, G={g_dn}) rows")
    assert_y_close(got[:, c3], ref_cols, rms, what=f"W2 ({c_dn.path}, G={g_dn}) cols")
