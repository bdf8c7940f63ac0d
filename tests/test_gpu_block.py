"""The block executor (w4a4_outlier_split_amd/block.py) on the device: per-module calibration
against the oracle's table builder and density, and the chained MLP through the executor checked
stage by stage against the oracle (each stage fed with the device's previous output)."""
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
from gpu_util import DEV, assert_y_close, codes_rm, dev_bits16, host_bits16, host_y, scales_rm  # noqa: E402


def dev_bf16(a):
    return dev_bits16(a).view(torch.bfloat16)


@pytest.mark.parametrize("gen", ["qkv", "attn_out", "ffn_down"])
def test_calibration_matches_the_oracle(gen):
    w = getattr(synth, gen)(S=16)
    cal = blk.calibrate(torch, dev_bf16(w.calib), w.H, 32)
    L, hits, ev = oracle.build_table(w.calib, 32)
    np.testing.assert_array_equal(cal.L[:, 0], L)
    np.testing.assert_array_equal(cal.hits[:, 0], hits)
    np.testing.assert_array_equal(cal.events, ev)
    assert cal.density == pytest.approx(oracle.mean_density(hits, ev), abs=1e-12)
    assert cal.path == ("fp8" if gen == "ffn_down" else "osc")


@pytest.mark.parametrize("down_path", ["fp8", "osc"])
def test_mlp_through_the_executor(down_path):
    S, H, F, G = 80, 512, 768, 32
    rng = np.random.default_rng(31)
    plant = synth.draw_plant(32, H, 0.6, 30.0, 80.0)
    X = synth.draw_x_bernoulli_spikes(S, H, plant, 33, None)
    cal = synth.draw_x_bernoulli_spikes(512, H, plant, 34, None)
    W13 = synth.draw_w(2 * F, H, 35)
    W2 = synth.draw_w(H, F, 36)
    c_up = blk.calibrate(torch, dev_bf16(cal), H, G)
    assert c_up.path == "osc"
    up = blk.Linear(torch, dev_bf16(W13), 2 * F, H, G, "osc", c_up.L)
    # the W2 table from the glue output of the calibration rows (the rule's own choice is fp8 on
    # this input; both paths are exercised)
    probe = blk.MLP(up, blk.Linear(torch, dev_bf16(W2), H, F, G, "fp8"))
    c_dn = probe.calibrate_down(torch, dev_bf16(cal), G)
    L2 = c_dn.L if down_path == "osc" else None
    down = blk.Linear(torch, dev_bf16(W2), H, F, G, down_path, L2)
    mlp = blk.MLP(up, down)
    bufs = mlp.buffers(S, DEV)
    Y = torch.empty((S, H), dtype=torch.float32, device=DEV)
    mlp.forward(dev_bf16(X), S, bufs, Y, osc.OSC_Y_F32)
    torch.cuda.synchronize()
    # calibration of W2 against the oracle on the device's own calibration glue output
    gu_cal = torch.empty((512, 2 * F), dtype=torch.bfloat16, device=DEV)
    up.forward(dev_bf16(cal), 512, up.act_buffers(512, DEV), gu_cal)
    torch.cuda.synchronize()
    h_cal = oracle.swiglu(host_bits16(gu_cal.view(torch.int16)))
    Lr, hr, er = oracle.build_table(h_cal, G)
    np.testing.assert_array_equal(c_dn.L[:, 0], Lr)
    assert c_dn.density == pytest.approx(oracle.mean_density(hr, er), abs=1e-12)
    # stage 1: the up-projection (bf16 output)
    GU = host_bits16(bufs["gu"].view(torch.int16))
    y1 = oracle.osc_linear(X, W13, G, c_up.L[:, 0])
    rel = np.abs(bits_to_f32(GU) - y1) / (np.abs(y1) + np.sqrt(np.mean(y1 ** 2)))
    assert rel.max() <= 2e-3 + 2 ** -8
    # stage 2: glue + quantization, bit for bit on the device's GU
    fmt = osc.OSC_MXFP4 if down_path == "osc" else osc.OSC_MXFP8
    rq, rs, rb = oracle.swiglu_quant(GU, G, None if L2 is None else L2, 1, fmt)
    QX, SX, B = bufs["h"]
    np.testing.assert_array_equal(codes_rm(QX, S, F, fmt), rq)
    np.testing.assert_array_equal(scales_rm(SX, S, F, G), rs)
    # stage 3: W2 at the usual tolerance
    if down_path == "osc":
        qw, sw, wl = oracle.pack_weights(W2, G, L2[:, 0])
        ref = oracle.gemm(rq, rs, qw, sw, G, rb, wl)
    else:
        qw, sw, _ = oracle.pack_weights(W2, G, None)
        ref = oracle.gemm(rq, rs, qw, sw, G, afmt=oracle.MXFP8, wfmt=oracle.MXFP4)
    assert_y_close(host_y(Y), ref, what=f"W2 ({down_path}) through the executor")


@pytest.mark.parametrize("gen", ["qkv", "attn_out"])
def test_group_size_rule_matches_the_oracle(gen):
    w = getattr(synth, gen)(S=16)
    G, shares = blk.calibrate_group_size(torch, dev_bf16(w.calib), w.H)
    ref = {g: blk.two_share(oracle.build_table_multi(w.calib, g, 2)[0]) for g in (64, 32, 16)}
    assert shares == pytest.approx(ref, abs=0)
    assert G == blk.choose_group_size(ref)
