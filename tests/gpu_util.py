"""Test-side helpers: move seeded numpy inputs to the GPU, run the libosc calls through the
Python binding, and compare against the oracle.  Outputs are pre-filled with 0xFF bytes
so that an unwritten element cannot pass a bit-exact comparison by accident."""
import numpy as np
import torch

import w4a4_outlier_split_amd as osc

DEV = "cuda:0"
Y_RTOL = 2e-3  # |dY| <= 2e-3 * (|Y| + RMS(Y)), per element


def dev_bits16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def poisoned(shape, dtype) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xFF)
    return t


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def code_cols(H: int, fmt: int) -> int:
    return H // 2 if fmt == osc.OSC_MXFP4 else H


def quant(X_dev: torch.Tensor, S: int, H: int, G: int, L, fmt: int):
    K = H // G
    QX = poisoned((S, code_cols(H, fmt)), torch.uint8)
    SX = poisoned((S, K), torch.uint8)
    B = poisoned((S, K), torch.int16) if L is not None else None
    osc.osc_quant_act(X_dev, S, H, G, L, fmt, QX, SX, B)
    return QX, SX, B


def pack(W_dev: torch.Tensor, N: int, H: int, G: int, L, fmt: int):
    K = H // G
    QW = poisoned((N, code_cols(H, fmt)), torch.uint8)
    SW = poisoned((N, K), torch.uint8)
    WL = poisoned((N, K), torch.int16) if L is not None else None
    osc.osc_pack_weights(W_dev, N, H, G, L, fmt, QW, SW, WL)
    return QW, SW, WL


def gemm(QX, SX, B, QW, SW, WL, S, N, H, G, yt=osc.OSC_Y_F32):
    Y = poisoned((S, N), torch.float32 if yt == osc.OSC_Y_F32 else torch.bfloat16)
    osc.osc_gemm(QX, SX, B, QW, SW, WL, S, N, H, G, Y, yt)
    return Y


def gemm_fp8(QX, SX, QW, SW, wfmt, S, N, H, G, yt=osc.OSC_Y_F32):
    Y = poisoned((S, N), torch.float32 if yt == osc.OSC_Y_F32 else torch.bfloat16)
    osc.osc_gemm_fp8(QX, SX, QW, SW, wfmt, S, N, H, G, Y, yt)
    return Y


def host_y(Y: torch.Tensor) -> np.ndarray:
    return Y.float().cpu().numpy().astype(np.float64)


def assert_y_close(got: np.ndarray, ref: np.ndarray, rms=None, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if rms is None:
        rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    bound = Y_RTOL * (np.abs(ref) + rms)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs outside tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    return float((err / bound).max())
