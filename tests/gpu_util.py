"""Test-side helpers: move seeded numpy inputs to the GPU, run the libosc calls through the
Python binding, and compare against the oracle.  Outputs are pre-filled with 0xFF bytes
so that an unwritten element cannot pass a bit-exact comparison by accident.

libosc's quantized operands use the tiled layout of include/osc.h; the oracle's are
row-major.  The ``*_rm`` helpers undo the tiling on the host (a pure permutation) so
the two compare element by element."""
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


def _tiled_outputs(R: int, H: int, G: int, fmt: int, with_side: bool, m: int = 1):
    Q = poisoned((osc.code_bytes(R, H, fmt),), torch.uint8)
    SC = poisoned((osc.scale_bytes(R, H, G, fmt),), torch.uint8)
    side = poisoned((osc.side_elems(R, H, G, m),), torch.int16) if with_side else None
    return Q, SC, side


def quant(X_dev: torch.Tensor, S: int, H: int, G: int, L, fmt: int):
    """-> tiled device buffers (QX, SX, B or None)."""
    QX, SX, B = _tiled_outputs(S, H, G, fmt, L is not None)
    osc.osc_quant_act(X_dev, S, H, G, L, fmt, QX, SX, B)
    return QX, SX, B


def pack(W_dev: torch.Tensor, N: int, H: int, G: int, L, fmt: int):
    """-> tiled device buffers (QW, SW, WL or None)."""
    QW, SW, WL = _tiled_outputs(N, H, G, fmt, L is not None)
    osc.osc_pack_weights(W_dev, N, H, G, L, fmt, QW, SW, WL)
    return QW, SW, WL


def quant_multi(X_dev: torch.Tensor, S: int, H: int, G: int, L, m: int, fmt: int = osc.OSC_MXFP4):
    """-> tiled device buffers (QX, SX, B with m*K compensation columns)."""
    QX, SX, B = _tiled_outputs(S, H, G, fmt, True, m)
    osc.osc_quant_act_multi(X_dev, S, H, G, L, m, fmt, QX, SX, B)
    return QX, SX, B


def pack_multi(W_dev: torch.Tensor, N: int, H: int, G: int, L, m: int, fmt: int = osc.OSC_MXFP4):
    QW, SW, WL = _tiled_outputs(N, H, G, fmt, True, m)
    osc.osc_pack_weights_multi(W_dev, N, H, G, L, m, fmt, QW, SW, WL)
    return QW, SW, WL


def gemm_multi(QX, SX, B, QW, SW, WL, S, N, H, G, m, yt=osc.OSC_Y_F32):
    Y = poisoned((S, N), torch.float32 if yt == osc.OSC_Y_F32 else torch.bfloat16)
    osc.osc_gemm_multi(QX, SX, B, QW, SW, WL, S, N, H, G, m, Y, yt)
    return Y


def codes_rm(t: torch.Tensor, R: int, H: int, fmt: int) -> np.ndarray:
    """tiled codes -> uint8[R, H/2 or H] row-major (panels of 128 channels)."""
    cb = 64 if fmt == osc.OSC_MXFP4 else 128
    a = host_u8(t).reshape(H // 128, R, cb)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(R, (H // 128) * cb))


def scales_rm(t: torch.Tensor, R: int, H: int, G: int) -> np.ndarray:
    """tiled E8M0 scales -> uint8[R, K] row-major (panels of 8 groups for G=16, else 4)."""
    K = H // G
    spg = 8 if G == 16 else 4
    a = host_u8(t).reshape(K // spg, R, spg)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(R, K))


def side_rm(t: torch.Tensor, R: int, H: int, G: int, m: int = 1) -> np.ndarray:
    """tiled B / W_L -> uint16 bf16 bits [R, m*K] row-major (panels of 32 columns)."""
    KC = m * (H // G)
    kp = (KC + 31) // 32
    a = host_bits16(t).reshape(kp, R, 32)
    return np.ascontiguousarray(a.transpose(1, 0, 2).reshape(R, kp * 32)[:, :KC])


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


def swiglu_quant(GU_dev: torch.Tensor, S: int, F: int, G: int, L, m: int, fmt: int):
    """-> tiled device buffers (QX, SX, B or None) of h = silu(gate) * up, GU = [gate | up]."""
    QX, SX, B = _tiled_outputs(S, F, G, fmt, L is not None, m)
    osc.osc_swiglu_quant(GU_dev, S, F, G, L, m, fmt, QX, SX, B)
    return QX, SX, B


def swiglu(GU_dev: torch.Tensor, S: int, F: int) -> torch.Tensor:
    Hh = poisoned((S, F), torch.int16)
    osc.osc_swiglu(GU_dev, S, F, Hh)
    return Hh


def linear_decode(X_dev: torch.Tensor, S: int, H: int, G: int, L, m: int, QW, SW, WL, N: int,
                  yt=osc.OSC_Y_F32) -> torch.Tensor:
    Y = poisoned((S, N), torch.float32 if yt == osc.OSC_Y_F32 else torch.bfloat16)
    osc.osc_linear_decode(X_dev, S, H, G, L, m, QW, SW, WL, N, Y, yt)
    return Y


def codes6_rm(t: torch.Tensor, R: int, H: int) -> np.ndarray:
    """tiled E3M2 pairs -> uint8[R, 3H/4] rows (element k at bits [6k, 6k+6)): per 128-channel
    stage, the R x 64 first region holds bytes 0..15 of block b's 24-byte fragment at [16b, 16b+16),
    the R x 32 second region bytes 16..23 at [8 * (b ^ (((r >> 1) ^ (r >> 3)) & 3)), +8)."""
    P = H // 128
    a = host_u8(t).reshape(P, R * 96)
    first = a[:, :R * 64].reshape(P, R, 4, 16)
    second = a[:, R * 64:].reshape(P, R, 4, 8)
    r = np.arange(R)[:, None]
    pos = np.arange(4)[None, :] ^ (((r >> 1) ^ (r >> 3)) & 3)          # [R, 4]: where block b's piece sits
    second = second[:, r, pos, :]                            # [P, R, 4, 8] in block order
    frag = np.concatenate([first, second], axis=3)           # [P, R, 4, 24]
    return np.ascontiguousarray(frag.transpose(1, 0, 2, 3).reshape(R, P * 96))


def gemm_fp6p(QX, SX, B, QW, SW, WL, S, N, H, m=1, yt=osc.OSC_Y_F32):
    Y = poisoned((S, N), torch.float32 if yt == osc.OSC_Y_F32 else torch.bfloat16)
    osc.osc_gemm_fp6p(QX, SX, B, QW, SW, WL, S, N, H, m, Y, yt)
    return Y
