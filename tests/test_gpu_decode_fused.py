"""GPU parity of osc_linear_decode (decode-sized batches, S <= 32: the activation quantization of
§3.2 fused into the skinny-S GEMM).  Its operands and accumulation order are those of
osc_quant_act_multi + osc_gemm_multi, so the bar is bit-for-bit equality with the two calls (fp32
and bf16 Y), plus the oracle's tolerance |dY| <= 2e-3 * (|Y| + RMS(Y))."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from gpu_util import (assert_y_close, dev_bits16, gemm_multi, host_y, linear_decode, pack, pack_multi,  # noqa: E402
                      quant, quant_multi)


def table(rng, K, G, m, p_none=0.25):
    L = np.full((K, m), -1, np.int32)
    for k in range(K):
        L[k] = np.where(rng.random(m) >= p_none, rng.choice(G, size=m, replace=False), -1)
    return L


CASES = [  # S, H, N, G, m (0: no table)
    (1, 256, 96, 32, 1), (7, 1024, 1000, 32, 1), (16, 1024, 520, 16, 2), (32, 512, 256, 64, 3),
    (13, 1024, 2080, 64, 1), (32, 4096, 600, 32, 0), (5, 768, 352, 16, 0), (16, 1024, 9000, 32, 3),
    (31, 2048, 17000, 16, 1), (2, 256, 64, 64, 2),
]


@pytest.mark.parametrize("S,H,N,G,m", CASES)
def test_fused_equals_the_two_calls_and_the_oracle(S, H, N, G, m):
    rng = np.random.default_rng(S * 1000 + H + N + G + m)
    X = synth.random_bf16((S, H), seed=S + H, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + G, scale=0.05)
    K = H // G
    L = table(rng, K, G, m) if m else None
    Xd, Wd = dev_bits16(X), dev_bits16(W)
    if m:
        QW, SW, WL = pack_multi(Wd, N, H, G, L, m)
        QX, SX, B = quant_multi(Xd, S, H, G, L, m)
    else:
        QW, SW, WL = pack(Wd, N, H, G, None, osc.OSC_MXFP4)
        QX, SX, B = quant(Xd, S, H, G, None, osc.OSC_MXFP4)
    for yt in (osc.OSC_Y_F32, osc.OSC_Y_BF16):
        Y2 = gemm_multi(QX, SX, B, QW, SW, WL, S, N, H, G, max(m, 1), yt)
        Yf = linear_decode(Xd, S, H, G, L, max(m, 1), QW, SW, WL, N, yt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Yf.cpu().view(torch.uint8).numpy(), Y2.cpu().view(torch.uint8).numpy())
    Yf = linear_decode(Xd, S, H, G, L, max(m, 1), QW, SW, WL, N)
    torch.cuda.synchronize()
    ref = oracle.osc_linear_multi(X, W, G, L, m) if m else oracle.osc_linear(X, W, G, None)
    assert_y_close(host_y(Yf), ref, what=f"fused decode S={S} H={H} N={N} G={G} m={m}")


def test_fused_ffn_up_decode_workload():
    """The FFN-up decode shape (S=16, H=4096, N=24576) with its built table: bit for bit the
    two-call result, and within tolerance of the oracle on 2048 sampled outputs."""
    w = synth.ffn_up(S=16)
    L, _, _ = oracle.build_table(w.calib, 32)
    Xd = dev_bits16(w.X)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, 32, L, osc.OSC_MXFP4)
    QX, SX, B = quant(Xd, w.S, w.H, 32, L, osc.OSC_MXFP4)
    Y2 = gemm_multi(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, 32, 1, osc.OSC_Y_BF16)
    Yf = linear_decode(Xd, w.S, w.H, 32, L, 1, QW, SW, WL, w.N, osc.OSC_Y_BF16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Yf.cpu().view(torch.int16).numpy(), Y2.cpu().view(torch.int16).numpy())
    cols = np.sort(np.random.default_rng(1).choice(w.N, 128, replace=False))
    Yf32 = linear_decode(Xd, w.S, w.H, 32, L, 1, QW, SW, WL, w.N, osc.OSC_Y_F32)
    torch.cuda.synchronize()
    ref = oracle.osc_linear(w.X, w.W[cols], 32, L)
    full = oracle.osc_linear(w.X[:2], w.W, 32, L)
    rms = float(np.sqrt(np.mean(full ** 2)))
    assert_y_close(host_y(Yf32)[:, cols], ref, rms=rms, what="fused FFN-up decode")
