"""GPU parity of the MLP glue of a Qwen3-shaped block (h = silu(gate) * up feeding W2, fused into
W2's input quantization) and of the chained MLP (W1/W3 up-projection -> glue -> W2) against the
oracle, through the C ABI.  h is defined as binary32 operations, so the bar is bit-exact: h itself
(osc_swiglu), and the codes, scales and B of osc_swiglu_quant.  The chain is checked stage by
stage (each oracle stage fed with the device's previous output) at the usual Y tolerance, and end
to end in norm."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import bits_to_f32, to_bf16_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402
from gpu_util import (assert_y_close, codes_rm, dev_bits16, gemm, gemm_fp8, host_bits16, host_y, pack,  # noqa: E402
                      quant, scales_rm, side_rm, swiglu, swiglu_quant)


def all_gate_patterns():
    """Every finite bf16 bit pattern once (non-finite ones replaced by +0), as 64 rows of 1024."""
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g[(g & 0x7F80) == 0x7F80] = 0
    return g.reshape(64, 1024)


@pytest.mark.parametrize("up", ["one", "random"])
def test_swiglu_h_bit_exact_over_every_gate_pattern(up):
    g = all_gate_patterns()
    S, F = g.shape
    if up == "one":
        u = np.full((S, F), 0x3F80, np.uint16)
    else:
        u = to_bf16_bits(np.clip(np.random.default_rng(9).normal(0, 0.6, (S, F)), -1, 1))
    GU = np.concatenate([g, u], axis=1)
    Hd = swiglu(dev_bits16(GU), S, F)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits16(Hd), oracle.swiglu(GU))


@pytest.mark.parametrize("fmt", [osc.OSC_MXFP4])
def test_swiglu_quant_h_inside_the_fused_kernel(fmt):
    """The fused kernel's h, seen through the compensation buffer: listing three channels per group
    copies h there bit for bit; eleven tables cover every channel of every gate pattern.  (Only the
    4-bit path takes a table; the E4M3 codes of h are checked without one below.)"""
    g = all_gate_patterns()
    S, F = g.shape
    G, m = 32, 3
    u = to_bf16_bits(np.clip(np.random.default_rng(10).normal(0, 0.6, (S, F)), -1, 1))
    GU = np.concatenate([g, u], axis=1)
    GUd = dev_bits16(GU)
    href = oracle.swiglu(GU)
    K = F // G
    for c0 in range(0, G, m):
        L = np.array([[c if c < G else -1 for c in (c0, c0 + 1, c0 + 2)]] * K, np.int32)
        QX, SX, B = swiglu_quant(GUd, S, F, G, L, m, fmt)
        torch.cuda.synchronize()
        rq, rs, rb = oracle.swiglu_quant(GU, G, L, m, fmt)
        np.testing.assert_array_equal(codes_rm(QX, S, F, fmt), rq)
        np.testing.assert_array_equal(scales_rm(SX, S, F, G), rs)
        got_b = side_rm(B, S, F, G, m)
        np.testing.assert_array_equal(got_b, rb)
        for e in range(m):
            if c0 + e < G:
                np.testing.assert_array_equal(got_b[:, e::m], href[:, c0 + e::G])


def test_swiglu_quant_e4m3_over_every_gate_pattern():
    """The FP8 fallback's input (no table): E4M3 codes and scales of h over every finite gate pattern."""
    g = all_gate_patterns()
    S, F = g.shape
    u = to_bf16_bits(np.clip(np.random.default_rng(11).normal(0, 0.6, (S, F)), -1, 1))
    GU = np.concatenate([g, u], axis=1)
    for G in (32, 64):
        QX, SX, _ = swiglu_quant(dev_bits16(GU), S, F, G, None, 1, osc.OSC_MXFP8)
        torch.cuda.synchronize()
        rq, rs, _ = oracle.swiglu_quant(GU, G, None, 1, oracle.MXFP8)
        np.testing.assert_array_equal(codes_rm(QX, S, F, osc.OSC_MXFP8), rq)
        np.testing.assert_array_equal(scales_rm(SX, S, F, G), rs)


@pytest.mark.parametrize("G", [16, 32, 64])
@pytest.mark.parametrize("fmt", [osc.OSC_MXFP4, osc.OSC_MXFP8])
@pytest.mark.parametrize("m", [0, 1, 2])
def test_swiglu_quant_ragged_rows(G, fmt, m):
    S, F = 37, 768
    rng = np.random.default_rng(G + 7 * m + 100 * fmt)
    GU = to_bf16_bits(rng.normal(0, 2.0, (S, 2 * F)))
    L = None
    if m:
        L = np.full((F // G, m), -1, np.int32)
        for k in range(F // G):
            L[k] = rng.choice(G, size=m, replace=False)
            if rng.random() < 0.2:
                L[k, -1] = -1
    if m and fmt == osc.OSC_MXFP8:
        # the FP8 fallback extracts nothing (no B / W_L in its GEMM): a table is refused
        with pytest.raises(osc.OscError) as e:
            swiglu_quant(dev_bits16(GU), S, F, G, L, m, fmt)
        assert e.value.status == 5  # OSC_E_FORMAT
        return
    QX, SX, B = swiglu_quant(dev_bits16(GU), S, F, G, L, max(m, 1), fmt)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.swiglu_quant(GU, G, L, max(m, 1), fmt)
    np.testing.assert_array_equal(codes_rm(QX, S, F, fmt), rq)
    np.testing.assert_array_equal(scales_rm(SX, S, F, G), rs)
    if m:
        np.testing.assert_array_equal(side_rm(B, S, F, G, m), rb)


def test_mlp_chain_stage_by_stage_and_end_to_end():
    """x -> OSC quant (table from calibration rows) -> up-projection [W1 | W3] (bf16 Y) -> glue fused
    into the FP8 quantization of W2's input -> W2 (MXFP4 weights, FP8 activations)."""
    S, H, F, G = 96, 512, 512, 32
    rng = np.random.default_rng(21)
    X = synth.random_bf16((S, H), seed=22)
    xv = bits_to_f32(X).astype(np.float64)
    cal = bits_to_f32(synth.random_bf16((256, H), seed=23)).astype(np.float64)
    for c in rng.choice(H, 10, replace=False):  # persistent channels, as in the workloads
        f = rng.uniform(40, 100)
        xv[:, c] *= f
        cal[:, c] *= f
    X, cal = to_bf16_bits(xv), to_bf16_bits(cal)
    W13 = synth.random_bf16((2 * F, H), seed=24, scale=0.02)
    W2 = synth.random_bf16((H, F), seed=25, scale=0.02)
    L, _, _ = oracle.build_table(cal, G)
    # stage 1: OSC up-projection, bf16 output
    QX, SX, B = quant(dev_bits16(X), S, H, G, L, osc.OSC_MXFP4)
    QW, SW, WL = pack(dev_bits16(W13), 2 * F, H, G, L, osc.OSC_MXFP4)
    GUd = gemm(QX, SX, B, QW, SW, WL, S, 2 * F, H, G, yt=osc.OSC_Y_BF16)
    # stage 2: glue + FP8 quantization of W2's input (no table: the fallback path of §4)
    Q8, S8, _ = swiglu_quant(GUd, S, F, G, None, 1, osc.OSC_MXFP8)
    # stage 3: W2 with MXFP4 weights
    QW2, SW2, _ = pack(dev_bits16(W2), H, F, G, None, osc.OSC_MXFP4)
    Y2 = gemm_fp8(Q8, S8, QW2, SW2, osc.OSC_MXFP4, S, H, F, G)
    torch.cuda.synchronize()
    GU = host_bits16(GUd)
    # stage 1 against the oracle, at the bf16 output's own rounding
    y1 = oracle.osc_linear(X, W13, G, L)
    assert np.max(np.abs(bits_to_f32(GU) - y1) / (np.abs(y1) + np.sqrt(np.mean(y1 ** 2)))) <= 2e-3 + 2 ** -8
    # stage 2 bit for bit on the device's own up-projection output
    rq, rs, _ = oracle.swiglu_quant(GU, G, None, 1, oracle.MXFP8)
    np.testing.assert_array_equal(codes_rm(Q8, S, F, osc.OSC_MXFP8), rq)
    np.testing.assert_array_equal(scales_rm(S8, S, F, G), rs)
    # stage 3 at the usual tolerance
    rqw, rsw, _ = oracle.pack_weights(W2, G, None, oracle.MXFP4)
    ref2 = oracle.gemm(rq, rs, rqw, rsw, G, afmt=oracle.MXFP8, wfmt=oracle.MXFP4)
    assert_y_close(host_y(Y2), ref2, what="W2 on the device's glue output")
    # end to end against the all-oracle chain (its own bf16-rounded up-projection): in norm
    GUo = to_bf16_bits(y1)
    q8o, s8o, _ = oracle.swiglu_quant(GUo, G, None, 1, oracle.MXFP8)
    refe = oracle.gemm(q8o, s8o, rqw, rsw, G, afmt=oracle.MXFP8, wfmt=oracle.MXFP4)
    assert np.linalg.norm(host_y(Y2) - refe) <= 2e-3 * np.linalg.norm(refe)
