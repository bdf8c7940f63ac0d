"""Python binding of libosc (include/osc.h): OSC W4A4 linear layers on MI355X (gfx950).

Argument marshalling only.  Every step runs in the HIP kernels of libosc.so;
there is no CPU fallback: importing this package fails loudly when the library
has not been built (``python w4a4_outlier_split_amd/build.py``).

Device buffers are torch tensors on a ROCm device (their ``data_ptr()`` is
passed through); table slices ``L`` are host arrays (numpy int32 or anything
``numpy.asarray`` accepts) or None.  ``stream=None`` means torch's current
stream on the current device.  A non-OK status raises :class:`OscError`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
# torch first: its HIP runtime must be the process's only one.  libosc's dependency on
# libamdhip64.so.7 then resolves to the runtime torch has already loaded; a second copy
# loaded ahead of torch does not see the device.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
# OSC_LIBRARY names another build of the same library (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("OSC_LIBRARY") or os.path.join(_HERE, "_build", "libosc.so")

OSC_MXFP4 = 0
OSC_MXFP8 = 1
OSC_FP6P = 2  # G = 16 pairs: E3M2 codes, one E8M0 scale per 32 channels
OSC_Y_BF16 = 0
OSC_Y_F32 = 1
OSC_MAX_GROUPS = 1024
OSC_MAX_CHANNELS = 3

STATUS = {0: "OSC_OK", 1: "OSC_E_NULL", 2: "OSC_E_SHAPE", 3: "OSC_E_TABLE", 4: "OSC_E_ALIGN",
          5: "OSC_E_FORMAT", 6: "OSC_E_DEVICE"}

EXPORTS = ("osc_pack_weights", "osc_quant_act", "osc_gemm", "osc_gemm_fp8", "osc_build_table",
           "osc_pack_weights_multi", "osc_quant_act_multi", "osc_gemm_multi", "osc_build_table_multi",
           "osc_swiglu_quant", "osc_swiglu", "osc_linear_decode", "osc_gemm_fp6p", "osc_status_str",
           "osc_last_device_error")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libosc.so is not built ({LIB_PATH}); run python w4a4_outlier_split_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double
_lib.osc_pack_weights.argtypes = [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P]
_lib.osc_quant_act.argtypes = [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P]
_lib.osc_gemm.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P]
_lib.osc_gemm_fp8.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P]
_lib.osc_build_table.argtypes = [_P, _I, _I, _I, _D, _D, _P, _P, _P, _P]
_lib.osc_pack_weights_multi.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P]
_lib.osc_quant_act_multi.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P]
_lib.osc_gemm_multi.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P]
_lib.osc_build_table_multi.argtypes = [_P, _I, _I, _I, _D, _D, _I, _P, _P, _P, _P]
_lib.osc_swiglu_quant.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P]
_lib.osc_swiglu.argtypes = [_P, _I, _I, _P, _P]
_lib.osc_linear_decode.argtypes = [_P, _I, _I, _I, _P, _I, _P, _P, _P, _I, _P, _I, _P]
_lib.osc_gemm_fp6p.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P]
for _f in EXPORTS[:-2]:
    getattr(_lib, _f).restype = _I
_lib.osc_status_str.argtypes = [_I]
_lib.osc_status_str.restype = ctypes.c_char_p
_lib.osc_last_device_error.argtypes = []
_lib.osc_last_device_error.restype = ctypes.c_char_p


def code_bytes(rows: int, H: int, fmt: int) -> int:
    """Bytes of a tiled code buffer (QX / QW) for ``rows`` rows of H channels."""
    return rows * (H // 2 if fmt == OSC_MXFP4 else H if fmt == OSC_MXFP8 else 3 * H // 4)


def scale_bytes(rows: int, H: int, G: int, fmt: int = OSC_MXFP4) -> int:
    """Bytes of a tiled E8M0 scale buffer (SX / SW): one per row and group (per pair of 16-groups
    for OSC_FP6P)."""
    return rows * (H // 32 if fmt == OSC_FP6P else H // G)


def side_elems(rows: int, H: int, G: int, m: int = 1) -> int:
    """bf16 elements of a tiled B / W_L buffer: m*K compensation columns in panels of 32, the
    last one padded."""
    return rows * ((m * (H // G) + 31) // 32) * 32


class OscError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = f"{call}: {osc_status_str(status)}"
        if status == 6:
            msg += f" ({_lib.osc_last_device_error().decode()})"
        super().__init__(msg)


def osc_status_str(status: int) -> str:
    return _lib.osc_status_str(int(status)).decode()


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int address), None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _table(L):
    if L is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(L), dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str) -> None:
    if status != 0:
        raise OscError(status, call)


def osc_pack_weights(W, N: int, H: int, G: int, L, wfmt: int, QW, SW, WL, stream=None) -> None:
    keep, lp = _table(L)
    _check(_lib.osc_pack_weights(_ptr(W), N, H, G, lp, wfmt, _ptr(QW), _ptr(SW), _ptr(WL), _stream(stream)),
           "osc_pack_weights")


def osc_quant_act(X, S: int, H: int, G: int, L, afmt: int, QX, SX, B, stream=None) -> None:
    keep, lp = _table(L)
    _check(_lib.osc_quant_act(_ptr(X), S, H, G, lp, afmt, _ptr(QX), _ptr(SX), _ptr(B), _stream(stream)),
           "osc_quant_act")


def osc_gemm(QX, SX, B, QW, SW, WL, S: int, N: int, H: int, G: int, Y, yt: int, stream=None) -> None:
    _check(_lib.osc_gemm(_ptr(QX), _ptr(SX), _ptr(B), _ptr(QW), _ptr(SW), _ptr(WL), S, N, H, G, _ptr(Y), yt,
                         _stream(stream)), "osc_gemm")


def osc_gemm_fp8(QX8, SX, QW, SW, wfmt: int, S: int, N: int, H: int, G: int, Y, yt: int, stream=None) -> None:
    _check(_lib.osc_gemm_fp8(_ptr(QX8), _ptr(SX), _ptr(QW), _ptr(SW), wfmt, S, N, H, G, _ptr(Y), yt,
                             _stream(stream)), "osc_gemm_fp8")


def osc_build_table(Xcal, R: int, H: int, G: int, alpha: float, rho: float, L, hits, events, stream=None) -> None:
    _check(_lib.osc_build_table(_ptr(Xcal), R, H, G, float(alpha), float(rho), _ptr(L), _ptr(hits), _ptr(events),
                                _stream(stream)), "osc_build_table")


# ---- several protected channels per group (L: m entries per group, [K, m] or flat K*m)

def osc_pack_weights_multi(W, N: int, H: int, G: int, L, m: int, wfmt: int, QW, SW, WL, stream=None) -> None:
    keep, lp = _table(L)
    _check(_lib.osc_pack_weights_multi(_ptr(W), N, H, G, lp, m, wfmt, _ptr(QW), _ptr(SW), _ptr(WL),
                                       _stream(stream)), "osc_pack_weights_multi")


def osc_quant_act_multi(X, S: int, H: int, G: int, L, m: int, afmt: int, QX, SX, B, stream=None) -> None:
    keep, lp = _table(L)
    _check(_lib.osc_quant_act_multi(_ptr(X), S, H, G, lp, m, afmt, _ptr(QX), _ptr(SX), _ptr(B), _stream(stream)),
           "osc_quant_act_multi")


def osc_swiglu_quant(GU, S: int, F: int, G: int, L, m: int, afmt: int, QX, SX, B, stream=None) -> None:
    """GU: [S, 2F] bf16 (gate | up) -> the tiled quantized h = silu(gate) * up (W2's input)."""
    keep, lp = _table(L)
    _check(_lib.osc_swiglu_quant(_ptr(GU), S, F, G, lp, m, afmt, _ptr(QX), _ptr(SX), _ptr(B), _stream(stream)),
           "osc_swiglu_quant")


def osc_gemm_fp6p(QX, SX, B, QW, SW, WL, S: int, N: int, H: int, m: int, Y, yt: int, stream=None) -> None:
    """G = 16 on E3M2 pairs (operands from the quant / pack calls with fmt OSC_FP6P, G = 16)."""
    _check(_lib.osc_gemm_fp6p(_ptr(QX), _ptr(SX), _ptr(B), _ptr(QW), _ptr(SW), _ptr(WL), S, N, H, m, _ptr(Y), yt,
                              _stream(stream)), "osc_gemm_fp6p")


def osc_linear_decode(X, S: int, H: int, G: int, L, m: int, QW, SW, WL, N: int, Y, yt: int, stream=None) -> None:
    """S <= 32: quantization of X fused into the GEMM; Y equals quant_act_multi + gemm_multi."""
    keep, lp = _table(L)
    _check(_lib.osc_linear_decode(_ptr(X), S, H, G, lp, m, _ptr(QW), _ptr(SW), _ptr(WL), N, _ptr(Y), yt,
                                  _stream(stream)), "osc_linear_decode")


def osc_swiglu(GU, S: int, F: int, Hout, stream=None) -> None:
    """GU: [S, 2F] bf16 (gate | up) -> Hout [S, F] bf16 = silu(gate) * up."""
    _check(_lib.osc_swiglu(_ptr(GU), S, F, _ptr(Hout), _stream(stream)), "osc_swiglu")


def osc_gemm_multi(QX, SX, B, QW, SW, WL, S: int, N: int, H: int, G: int, m: int, Y, yt: int, stream=None) -> None:
    _check(_lib.osc_gemm_multi(_ptr(QX), _ptr(SX), _ptr(B), _ptr(QW), _ptr(SW), _ptr(WL), S, N, H, G, m, _ptr(Y),
                               yt, _stream(stream)), "osc_gemm_multi")


def osc_build_table_multi(Xcal, R: int, H: int, G: int, alpha: float, rho: float, m: int, L, hits, events,
                          stream=None) -> None:
    _check(_lib.osc_build_table_multi(_ptr(Xcal), R, H, G, float(alpha), float(rho), m, _ptr(L), _ptr(hits),
                                      _ptr(events), _stream(stream)), "osc_build_table_multi")
