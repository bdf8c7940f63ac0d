"""GPU parity of the HIP path against the CPU oracle, through the C ABI (Python binding).

Bar: element codes, E8M0 scales, B and W_L bit-exact; table slices exact; Y within
|dY| <= 2e-3 * (|Y| + RMS(Y)) per element, RMS over the compared oracle outputs.
Full-size workloads compare every quantized byte and sampled GEMM outputs (rows /
columns the oracle computes one by one), in the launch configurations the benchmark uses.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import bits_to_f32, to_bf16_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import w4a4_outlier_split_amd as osc  # noqa: E402  (loud ImportError when the library is missing)
from gpu_util import (assert_y_close, codes_rm, dev_bits16, gemm, gemm_fp8, host_y, pack, quant,  # noqa: E402
                      scales_rm, side_rm)

FP4, FP8 = osc.OSC_MXFP4, osc.OSC_MXFP8


@functools.lru_cache(maxsize=None)
def workload(name):
    if name == "tiny":
        return synth.tiny()
    if name == "qkv":
        return synth.qkv(S=2048)
    if name == "ffn_up":
        return synth.ffn_up(S=4096)
    if name == "ffn_down":
        return synth.ffn_down(S=4096)
    if name.startswith("gsweep"):
        _, s, g = name.split("_")
        return synth.group_sweep(int(s), int(g))
    raise KeyError(name)


@functools.lru_cache(maxsize=None)
def table(name):
    w = workload(name)
    if w.L is not None:
        return w.L
    L, _, _ = oracle.build_table(w.calib, w.G)
    return L


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist())
    idx.update({0, n - 1})
    return np.array(sorted(idx))


# ------------------------------------------------------------------ quantization

@pytest.mark.parametrize("G", [16, 32, 64])
@pytest.mark.parametrize("fmt", [FP4, FP8])
def test_quant_exhaustive_bf16(G, fmt):
    """Every finite bf16 pattern, in several arrangements (so each meets many group scales)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(bits_to_f32(bits))
    bits = np.where(finite, bits, 0).astype(np.uint16)
    rng = np.random.default_rng(G + fmt)
    rows = [bits, bits[::-1].copy()] + [rng.permutation(bits) for _ in range(4)]
    X = np.stack(rows).reshape(-1, 8192)  # K = 8192 / G stays within OSC_MAX_GROUPS
    S, H = X.shape
    K = H // G
    L = rng.integers(-1, G, K).astype(np.int32) if fmt == FP4 else None
    QX, SX, B = quant(dev_bits16(X), S, H, G, L, fmt)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act(X, G, L, fmt)
    np.testing.assert_array_equal(scales_rm(SX, S, H, G), rs)
    np.testing.assert_array_equal(codes_rm(QX, S, H, fmt), rq)
    if L is not None:
        np.testing.assert_array_equal(side_rm(B, S, H, G), rb)


@pytest.mark.parametrize("name", ["tiny", "qkv", "gsweep_8192_16", "gsweep_2048_64"])
def test_quant_workloads_mxfp4(name):
    w = workload(name)
    L = table(name)
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    torch.cuda.synchronize()
    rq, rs, rb = oracle.quant_act(w.X, w.G, L, FP4)
    np.testing.assert_array_equal(scales_rm(SX, w.S, w.H, w.G), rs)
    np.testing.assert_array_equal(side_rm(B, w.S, w.H, w.G), rb)
    np.testing.assert_array_equal(codes_rm(QX, w.S, w.H, FP4), rq)


def test_quant_down_proj_mxfp8():
    w = workload("ffn_down")
    QX, SX, _ = quant(dev_bits16(w.X), w.S, w.H, w.G, None, FP8)
    torch.cuda.synchronize()
    rows = sample_rows(w.S, 512, 1)
    rq, rs, _ = oracle.quant_act(w.X[rows], w.G, None, FP8)
    np.testing.assert_array_equal(scales_rm(SX, w.S, w.H, w.G)[rows], rs)
    np.testing.assert_array_equal(codes_rm(QX, w.S, w.H, FP8)[rows], rq)


def test_quant_ragged_and_empty():
    """37 rows (no tile multiple), K = 4 .. 16 groups (scale panels, a partial B panel)."""
    S, H = 37, 256
    X = synth.random_bf16((S, H), seed=5, scale=3.0)
    L = np.array([5, -1, 0, 15, 15, -1, 3, 3, 0, 1, 2, -1, 7, 8, 9, 10], np.int32)
    for G, Lg, fmt in ((16, L, FP4), (32, L[:8], FP4), (32, None, FP4), (64, L[:4], FP4), (64, None, FP8)):
        QX, SX, B = quant(dev_bits16(X), S, H, G, Lg, fmt)
        torch.cuda.synchronize()
        rq, rs, rb = oracle.quant_act(X, G, Lg, fmt)
        np.testing.assert_array_equal(codes_rm(QX, S, H, fmt), rq)
        np.testing.assert_array_equal(scales_rm(SX, S, H, G), rs)
        if Lg is not None:
            np.testing.assert_array_equal(side_rm(B, S, H, G), rb)
    # S = 0: valid, launches nothing
    empty = torch.empty((0, 256), dtype=torch.int16, device="cuda:0")
    osc.osc_quant_act(empty, 0, 256, 32, None, FP4, empty, empty, None)


# ------------------------------------------------------------------ weight packing

@pytest.mark.parametrize("name,fmt", [("tiny", FP4), ("qkv", FP4), ("ffn_up", FP4), ("ffn_down", FP4),
                                      ("ffn_down", FP8), ("gsweep_16_16", FP4), ("gsweep_16_64", FP4)])
def test_pack_weights(name, fmt):
    w = workload(name)
    L = table(name) if fmt == FP4 else None  # MXFP8 weights serve the FP8 fallback: no W_L
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, fmt)
    torch.cuda.synchronize()
    rows = sample_rows(w.N, 1024, 2)
    rq, rs, rwl = oracle.pack_weights(w.W[rows], w.G, L, fmt)
    np.testing.assert_array_equal(scales_rm(SW, w.N, w.H, w.G)[rows], rs)
    np.testing.assert_array_equal(codes_rm(QW, w.N, w.H, fmt)[rows], rq)
    if L is not None:
        np.testing.assert_array_equal(side_rm(WL, w.N, w.H, w.G)[rows], rwl)


# ------------------------------------------------------------------ table builder

@pytest.mark.parametrize("name,G", [("qkv", 32), ("qkv", 16), ("qkv", 64), ("ffn_down", 32)])
def test_build_table(name, G):
    w = workload(name)
    K = w.H // G
    out = [torch.full((K,), -7, dtype=torch.int32, device="cuda:0") for _ in range(3)]
    osc.osc_build_table(dev_bits16(w.calib), w.calib.shape[0], w.H, G, 5.0, 0.35, *out)
    torch.cuda.synchronize()
    L, hits, events = oracle.build_table(w.calib, G, 5.0, 0.35)
    np.testing.assert_array_equal(out[0].cpu().numpy(), L)
    np.testing.assert_array_equal(out[1].cpu().numpy(), hits)
    np.testing.assert_array_equal(out[2].cpu().numpy(), events)


# ------------------------------------------------------------------ dual-path GEMM

def run_osc(w, L, rows, cols, yt=osc.OSC_Y_F32, comp=True):
    L = L if comp else None  # without compensation nothing is extracted either (direct MXFP4)
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G, yt)
    torch.cuda.synchronize()
    got = host_y(Y)
    rq, rs, rb = oracle.quant_act(w.X[rows], w.G, L, FP4)
    wq, ws, wl = oracle.pack_weights(w.W[cols], w.G, L, FP4)
    ref = oracle.gemm(rq, rs, wq, ws, w.G, rb, wl)
    return got, ref


def test_gemm_tiny_full():
    w = workload("tiny")
    L = table("tiny")
    allr, allc = np.arange(w.S), np.arange(w.N)
    got, ref = run_osc(w, L, allr, allc)
    assert_y_close(got, ref, what="tiny")
    got, ref = run_osc(w, L, allr, allc, comp=False)
    assert_y_close(got, ref, what="tiny, no compensation")


@pytest.mark.parametrize("name", ["tiny", "qkv"])
def test_gemm_bf16_output_is_rne_of_fp32(name):
    """The tolerance is stated on the fp32 result; a bf16 output adds only its own rounding
    (up to 2^-8 |Y|), so it must be exactly the round-to-nearest-even of the fp32 result."""
    w = workload(name)
    L = table(name)
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    Yf = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G, osc.OSC_Y_F32)
    Yb = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G, osc.OSC_Y_BF16)
    torch.cuda.synchronize()
    assert torch.equal(Yb.view(torch.int16), Yf.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("name", ["qkv", "ffn_up", "gsweep_8192_16", "gsweep_8192_32", "gsweep_8192_64"])
def test_gemm_workloads_sampled(name):
    w = workload(name)
    L = table(name)
    rows = sample_rows(w.S, 24, 3)
    wide = sample_rows(w.N, 2048, 8)
    cols = sample_rows(w.N, 24, 4)
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G)
    torch.cuda.synchronize()
    got = host_y(Y)
    rq, rs, rb = oracle.quant_act(w.X[rows], w.G, L, FP4)
    wq, ws, wl = oracle.pack_weights(w.W[wide], w.G, L, FP4)
    ref_rows = oracle.gemm(rq, rs, wq, ws, w.G, rb, wl)            # sampled rows x 2048 columns
    xq, xs, xb = oracle.quant_act(w.X, w.G, L, FP4)
    cq, cs, cl = oracle.pack_weights(w.W[cols], w.G, L, FP4)
    ref_cols = oracle.gemm(xq, xs, cq, cs, w.G, xb, cl)             # every row, sampled columns
    rms = float(np.sqrt(np.mean(ref_rows ** 2)))
    assert_y_close(got[np.ix_(rows, wide)], ref_rows, rms, what=f"{name} rows")
    assert_y_close(got[:, cols], ref_cols, rms, what=f"{name} cols")


@pytest.mark.parametrize("S", [16, 1, 77])
def test_gemm_decode_and_ragged_rows(S):
    w = workload("ffn_up")
    L = table("ffn_up")
    X = w.X[:S]
    cols = sample_rows(w.N, 512, 5)
    QX, SX, B = quant(dev_bits16(X), S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, S, w.N, w.H, w.G)
    torch.cuda.synchronize()
    got = host_y(Y)[:, cols]
    rq, rs, rb = oracle.quant_act(X, w.G, L, FP4)
    wq, ws, wl = oracle.pack_weights(w.W[cols], w.G, L, FP4)
    assert_y_close(got, oracle.gemm(rq, rs, wq, ws, w.G, rb, wl), what=f"S={S}")


@pytest.mark.parametrize("S,N,H,G", [(77, 200, 512, 32), (130, 72, 256, 16), (33, 300, 512, 64), (5, 1, 256, 32)])
def test_gemm_ragged_shapes(S, N, H, G):
    X = synth.random_bf16((S, H), seed=S, scale=2.0)
    W = synth.random_bf16((N, H), seed=N, scale=0.05)
    L = np.random.default_rng(H + G).integers(-1, G, H // G).astype(np.int32)
    QX, SX, B = quant(dev_bits16(X), S, H, G, L, FP4)
    QW, SW, WL = pack(dev_bits16(W), N, H, G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, S, N, H, G)
    torch.cuda.synchronize()
    ref = oracle.osc_linear(X, W, G, L)
    assert_y_close(host_y(Y), ref, what=f"{S}x{N}x{H} G={G}")


def test_all_minus_one_table_is_plain_mxfp4():
    w = workload("tiny")
    L = np.full(w.H // w.G, -1, np.int32)
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    assert np.all(side_rm(B, w.S, w.H, w.G) == 0) and np.all(side_rm(WL, w.N, w.H, w.G) == 0)
    Y1 = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G)
    QX2, SX2, _ = quant(dev_bits16(w.X), w.S, w.H, w.G, None, FP4)
    assert torch.equal(QX, QX2) and torch.equal(SX, SX2)
    Y2 = gemm(QX2, SX2, None, QW, SW, None, w.S, w.N, w.H, w.G)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_gemm_deterministic():
    w = workload("qkv")
    L = table("qkv")
    QX, SX, B = quant(dev_bits16(w.X), w.S, w.H, w.G, L, FP4)
    QW, SW, WL = pack(dev_bits16(w.W), w.N, w.H, w.G, L, FP4)
    Y1 = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G, osc.OSC_Y_BF16)
    Y2 = gemm(QX, SX, B, QW, SW, WL, w.S, w.N, w.H, w.G, osc.OSC_Y_BF16)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


# ------------------------------------------------------------------ FP8 fallback (W2)

@pytest.mark.parametrize("wfmt", [FP4, FP8])
def test_gemm_fp8_down_proj(wfmt):
    w = workload("ffn_down")
    rows = sample_rows(w.S, 16, 6)
    wide = sample_rows(w.N, 1024, 9)
    cols = sample_rows(w.N, 16, 7)
    QX, SX, _ = quant(dev_bits16(w.X), w.S, w.H, w.G, None, FP8)
    QW, SW, _ = pack(dev_bits16(w.W), w.N, w.H, w.G, None, wfmt)
    Y = gemm_fp8(QX, SX, QW, SW, wfmt, w.S, w.N, w.H, w.G)
    torch.cuda.synchronize()
    got = host_y(Y)
    rq, rs, _ = oracle.quant_act(w.X[rows], w.G, None, FP8)
    wq, ws, _ = oracle.pack_weights(w.W[wide], w.G, None, wfmt)
    ref_rows = oracle.gemm(rq, rs, wq, ws, w.G, afmt=FP8, wfmt=wfmt)
    xq, xs, _ = oracle.quant_act(w.X, w.G, None, FP8)
    cq, cs, _ = oracle.pack_weights(w.W[cols], w.G, None, wfmt)
    ref_cols = oracle.gemm(xq, xs, cq, cs, w.G, afmt=FP8, wfmt=wfmt)
    rms = float(np.sqrt(np.mean(ref_rows ** 2)))
    assert_y_close(got[np.ix_(rows, wide)], ref_rows, rms, what="fp8 rows")
    assert_y_close(got[:, cols], ref_cols, rms, what="fp8 cols")


@pytest.mark.parametrize("S,N,H,G,wfmt", [(77, 200, 512, 32, FP4), (9, 72, 256, 64, FP8), (130, 40, 768, 32, FP8)])
def test_gemm_fp8_ragged(S, N, H, G, wfmt):
    X = synth.random_bf16((S, H), seed=S + 1, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + 1, scale=0.05)
    QX, SX, _ = quant(dev_bits16(X), S, H, G, None, FP8)
    QW, SW, _ = pack(dev_bits16(W), N, H, G, None, wfmt)
    Y = gemm_fp8(QX, SX, QW, SW, wfmt, S, N, H, G)
    torch.cuda.synchronize()
    rq, rs, _ = oracle.quant_act(X, G, None, FP8)
    wq, ws, _ = oracle.pack_weights(W, G, None, wfmt)
    assert_y_close(host_y(Y), oracle.gemm(rq, rs, wq, ws, G, afmt=FP8, wfmt=wfmt), what=f"fp8 {S}x{N}x{H}")


# ------------------------------------------------------------------ skinny-S (decode) kernel

@pytest.mark.parametrize("S", [1, 9, 16, 17, 32])
@pytest.mark.parametrize("G,comp", [(16, True), (32, True), (32, False), (64, True)])
def test_gemm_decode_kernel(S, G, comp):
    """S <= 32 runs the skinny-S kernel (K split over the waves of a 32-column block); S = 9 and 16
    leave rows of the 32-row MFMA blocks unused."""
    N, H = 300, 1536  # ragged last column block; 12 main stages over 8 waves
    X = synth.random_bf16((S, H), seed=S * 7 + G, scale=2.0)
    W = synth.random_bf16((N, H), seed=G + 3, scale=0.05)
    L = np.random.default_rng(S + G).integers(-1, G, H // G).astype(np.int32) if comp else None
    QX, SX, B = quant(dev_bits16(X), S, H, G, L, FP4)
    QW, SW, WL = pack(dev_bits16(W), N, H, G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, S, N, H, G)
    Yb = gemm(QX, SX, B, QW, SW, WL, S, N, H, G, osc.OSC_Y_BF16)
    torch.cuda.synchronize()
    ref = oracle.osc_linear(X, W, G, L) if comp else oracle.gemm(*oracle.quant_act(X, G, None)[:2],
                                                                *oracle.pack_weights(W, G, None)[:2], G)
    assert_y_close(host_y(Y), ref, what=f"decode S={S} G={G} comp={comp}")
    assert torch.equal(Yb.view(torch.int16), Y.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("S,wfmt,G", [(16, FP4, 32), (7, FP8, 64), (32, FP4, 64)])
def test_gemm_fp8_decode_kernel(S, wfmt, G):
    N, H = 200, 1536
    X = synth.random_bf16((S, H), seed=S + 11, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + 12, scale=0.05)
    QX, SX, _ = quant(dev_bits16(X), S, H, G, None, FP8)
    QW, SW, _ = pack(dev_bits16(W), N, H, G, None, wfmt)
    Y = gemm_fp8(QX, SX, QW, SW, wfmt, S, N, H, G)
    torch.cuda.synchronize()
    rq, rs, _ = oracle.quant_act(X, G, None, FP8)
    wq, ws, _ = oracle.pack_weights(W, G, None, wfmt)
    assert_y_close(host_y(Y), oracle.gemm(rq, rs, wq, ws, G, afmt=FP8, wfmt=wfmt), what=f"fp8 decode S={S}")


@pytest.mark.parametrize("S,N,H,G", [(1024, 8192, 1024, 32),   # 256x128 tiles
                                     (512, 8192, 512, 64),     # 128x128 tiles
                                     (2048, 6144, 1024, 16)])  # 256x192 tiles at G=16
def test_gemm_every_tile_shape(S, N, H, G):
    """Shapes that make the tile choice pick each prefill configuration; sampled rows x all columns
    and all rows x sampled columns against the oracle."""
    X = synth.random_bf16((S, H), seed=S + H, scale=2.0)
    W = synth.random_bf16((N, H), seed=N + H, scale=0.05)
    L = np.random.default_rng(G + H).integers(-1, G, H // G).astype(np.int32)
    QX, SX, B = quant(dev_bits16(X), S, H, G, L, FP4)
    QW, SW, WL = pack(dev_bits16(W), N, H, G, L, FP4)
    Y = gemm(QX, SX, B, QW, SW, WL, S, N, H, G)
    torch.cuda.synchronize()
    got = host_y(Y)
    rows = sample_rows(S, 12, 31)
    cols = sample_rows(N, 12, 32)
    wide = sample_rows(N, 1024, 33)
    rq, rs, rb = oracle.quant_act(X[rows], G, L, FP4)
    wq, ws, wl = oracle.pack_weights(W[wide], G, L, FP4)
    ref_rows = oracle.gemm(rq, rs, wq, ws, G, rb, wl)
    xq, xs, xb = oracle.quant_act(X, G, L, FP4)
    cq, cs, cl = oracle.pack_weights(W[cols], G, L, FP4)
    ref_cols = oracle.gemm(xq, xs, cq, cs, G, xb, cl)
    rms = float(np.sqrt(np.mean(ref_rows ** 2)))
    assert_y_close(got[np.ix_(rows, wide)], ref_rows, rms, what=f"{S}x{N}x{H} G={G} rows")
    assert_y_close(got[:, cols], ref_cols, rms, what=f"{S}x{N}x{H} G={G} cols")


@pytest.mark.parametrize("m", [1, 2])
def test_build_table_ties_and_alpha_boundary(m):
    """Hand-built calibration groups (in-row arg-max ties, a max exactly on alpha * mean): the device
    builder equals the oracle and the hand-derived table."""
    import calib_cases as cc
    R = 64
    cal = to_bf16_bits(cc.calibration_rows(R))
    H = cal.shape[1]
    K = H // cc.G
    L = torch.full((K * m,), -7, dtype=torch.int32, device="cuda:0")
    hits = torch.full((K * m,), -7, dtype=torch.int32, device="cuda:0")
    ev = torch.full((K,), -7, dtype=torch.int32, device="cuda:0")
    osc.osc_build_table_multi(dev_bits16(cal), R, H, cc.G, cc.ALPHA, cc.RHO, m, L, hits, ev)
    torch.cuda.synchronize()
    rL, rh, re = oracle.build_table_multi(cal, cc.G, m, cc.ALPHA, cc.RHO)
    got = L.cpu().numpy().reshape(K, m)
    np.testing.assert_array_equal(got, rL)
    np.testing.assert_array_equal(hits.cpu().numpy().reshape(K, m), rh)
    np.testing.assert_array_equal(ev.cpu().numpy(), re)
    np.testing.assert_array_equal(got.reshape(-1) if m == 1 else got, cc.expected(m))
