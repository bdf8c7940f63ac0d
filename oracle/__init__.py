"""CPU oracle for OSC W4A4 linear layers -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The arithmetic lives in ``osc_oracle.c`` (plain
C, fp64); this module only marshals numpy arrays through ctypes.  See that
file's header for the passages of the OSC page each function follows.

All bf16 data is passed as raw bit patterns (``numpy.uint16``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

MXFP4 = 0
MXFP8 = 1
FP6P = 2  # E3M2 codes, one E8M0 scale per pair of 16-groups

_lib = None


def lib():
    global _lib
    if _lib is None:
        # OSC_ORACLE_LIBRARY names another build of osc_oracle.c (the sanitizer build of the tests)
        path = os.environ.get("OSC_ORACLE_LIBRARY")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_scale_exp.argtypes = [ctypes.c_double, i]
        L.orc_scale_exp.restype = i
        L.orc_quant_act.argtypes = [P, i, i, i, P, i, P, P, P]
        L.orc_quant_act.restype = None
        L.orc_pack_weights.argtypes = [P, i, i, i, P, i, P, P, P]
        L.orc_pack_weights.restype = None
        L.orc_gemm.argtypes = [P, P, i, P, P, P, i, P, i, i, i, i, P]
        L.orc_gemm.restype = None
        L.orc_build_table.argtypes = [P, i, i, i, ctypes.c_double, ctypes.c_double, P, P, P]
        L.orc_build_table.restype = i
        L.orc_gemm_comp.argtypes = [P, P, i, P, P, P, i, P, i, i, i, i, i, P]
        L.orc_gemm_comp.restype = None
        L.orc_quant_act_multi.argtypes = [P, i, i, i, P, i, i, P, P, P]
        L.orc_quant_act_multi.restype = None
        L.orc_pack_weights_multi.argtypes = [P, i, i, i, P, i, i, P, P, P]
        L.orc_pack_weights_multi.restype = None
        L.orc_build_table_multi.argtypes = [P, i, i, i, ctypes.c_double, ctypes.c_double, i, P, P, P]
        L.orc_build_table_multi.restype = i
        L.orc_threads.argtypes = []
        L.orc_threads.restype = i
        L.orc_exp32.argtypes = [ctypes.c_float]
        L.orc_exp32.restype = ctypes.c_float
        L.orc_silu32.argtypes = [ctypes.c_float]
        L.orc_silu32.restype = ctypes.c_float
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_swiglu.argtypes = [P, i, i, P]
        L.orc_swiglu.restype = None
        L.orc_mean_density.argtypes = [P, P, i, i]
        L.orc_mean_density.restype = ctypes.c_double
        L.orc_e3m2_decode.argtypes = [ctypes.c_uint8]
        L.orc_e3m2_decode.restype = ctypes.c_double
        L.orc_e3m2_encode.argtypes = [ctypes.c_double]
        L.orc_e3m2_encode.restype = ctypes.c_uint8
        L.orc_quant_act_fp6p.argtypes = [P, i, i, P, i, P, P, P]
        L.orc_quant_act_fp6p.restype = None
        L.orc_pack_weights_fp6p.argtypes = [P, i, i, P, i, P, P, P]
        L.orc_pack_weights_fp6p.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_threads())


# ------------------------------------------------------------ scalar codecs

def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code))


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(int(code))


def e2m1_encode(v: float) -> int:
    return int(lib().orc_e2m1_encode(float(v)))


def e4m3_encode(v: float) -> int:
    return int(lib().orc_e4m3_encode(float(v)))


def scale_exp(amax: float, fmt: int) -> int:
    return int(lib().orc_scale_exp(float(amax), int(fmt)))


# ------------------------------------------------------------ array entry points

def code_bytes_per_row(H: int, fmt: int) -> int:
    return H // 2 if fmt == MXFP4 else H if fmt == MXFP8 else 3 * H // 4


def quant_act(X: np.ndarray, G: int, L: Optional[np.ndarray], fmt: int = MXFP4
              ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """X: uint16[S, H] bf16 bits -> (QX uint8[S, H/2 or H], SX uint8[S, K], B uint16[S, K] or None)."""
    X = _c(X, np.uint16)
    S, H = X.shape
    K = H // G
    QX = np.zeros((S, code_bytes_per_row(H, fmt)), np.uint8)
    SX = np.zeros((S, K), np.uint8)
    Lc = None if L is None else _c(L, np.int32)
    B = None if L is None else np.zeros((S, K), np.uint16)
    lib().orc_quant_act(_p(X), S, H, G, _p(Lc), fmt, _p(QX), _p(SX), _p(B))
    return QX, SX, B


def pack_weights(W: np.ndarray, G: int, L: Optional[np.ndarray], fmt: int = MXFP4
                 ) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """W: uint16[N, H] bf16 bits -> (QW, SW uint8[N, K], WL uint16[N, K] or None)."""
    W = _c(W, np.uint16)
    N, H = W.shape
    K = H // G
    QW = np.zeros((N, code_bytes_per_row(H, fmt)), np.uint8)
    SW = np.zeros((N, K), np.uint8)
    Lc = None if L is None else _c(L, np.int32)
    WL = None if L is None else np.zeros((N, K), np.uint16)
    lib().orc_pack_weights(_p(W), N, H, G, _p(Lc), fmt, _p(QW), _p(SW), _p(WL))
    return QW, SW, WL


def gemm(QX, SX, QW, SW, G: int, B=None, WL=None, afmt: int = MXFP4, wfmt: int = MXFP4) -> np.ndarray:
    """Dual-path GEMM in fp64 -> float64[S, N]."""
    QX = _c(QX, np.uint8)
    SX = _c(SX, np.uint8)
    QW = _c(QW, np.uint8)
    SW = _c(SW, np.uint8)
    S = QX.shape[0]
    N = QW.shape[0]
    H = SX.shape[1] * G
    assert QX.shape[1] == code_bytes_per_row(H, afmt) and QW.shape[1] == code_bytes_per_row(H, wfmt)
    Bc = None if B is None else _c(B, np.uint16)
    WLc = None if WL is None else _c(WL, np.uint16)
    Y = np.zeros((S, N), np.float64)
    lib().orc_gemm(_p(QX), _p(SX), afmt, _p(Bc), _p(QW), _p(SW), wfmt, _p(WLc), S, N, H, G, _p(Y))
    return Y


def build_table(Xcal: np.ndarray, G: int, alpha: float = 5.0, rho: float = 0.35):
    """Algorithm 1 reading -> (L int32[K], hits int32[K], events int32[K])."""
    Xcal = _c(Xcal, np.uint16)
    R, H = Xcal.shape
    K = H // G
    L = np.zeros(K, np.int32)
    hits = np.zeros(K, np.int32)
    events = np.zeros(K, np.int32)
    lib().orc_build_table(_p(Xcal), R, H, G, float(alpha), float(rho), _p(L), _p(hits), _p(events))
    return L, hits, events


def osc_linear(X, W, G: int, L, fmt: int = MXFP4):
    """Convenience: quant_act + pack_weights + gemm (the whole OSC layer) in fp64."""
    QX, SX, B = quant_act(X, G, L, fmt)
    QW, SW, WL = pack_weights(W, G, L, MXFP4 if fmt == MXFP8 else fmt)
    return gemm(QX, SX, QW, SW, G, B, WL, afmt=fmt, wfmt=MXFP4 if fmt == MXFP8 else fmt)


# ------------------------------------------------ several channels per group (§6)

def quant_act_multi(X: np.ndarray, G: int, L: np.ndarray, m: int, fmt: int = MXFP4):
    """L: int32[K, m] (or K*m flat) -> (QX, SX uint8[S, K], B uint16[S, K*m])."""
    X = _c(X, np.uint16)
    S, H = X.shape
    K = H // G
    Lc = _c(L, np.int32).reshape(K * m)
    QX = np.zeros((S, code_bytes_per_row(H, fmt)), np.uint8)
    SX = np.zeros((S, K), np.uint8)
    B = np.zeros((S, K * m), np.uint16)
    lib().orc_quant_act_multi(_p(X), S, H, G, _p(Lc), m, fmt, _p(QX), _p(SX), _p(B))
    return QX, SX, B


def pack_weights_multi(W: np.ndarray, G: int, L: np.ndarray, m: int, fmt: int = MXFP4):
    """-> (QW, SW uint8[N, K], WL uint16[N, K*m])."""
    W = _c(W, np.uint16)
    N, H = W.shape
    K = H // G
    Lc = _c(L, np.int32).reshape(K * m)
    QW = np.zeros((N, code_bytes_per_row(H, fmt)), np.uint8)
    SW = np.zeros((N, K), np.uint8)
    WL = np.zeros((N, K * m), np.uint16)
    lib().orc_pack_weights_multi(_p(W), N, H, G, _p(Lc), m, fmt, _p(QW), _p(SW), _p(WL))
    return QW, SW, WL


def gemm_comp(QX, SX, QW, SW, G: int, B, WL, afmt: int = MXFP4, wfmt: int = MXFP4) -> np.ndarray:
    """Dual-path GEMM with B / WL of any number of compensation columns (S x KC, N x KC)."""
    QX, SX, QW, SW = _c(QX, np.uint8), _c(SX, np.uint8), _c(QW, np.uint8), _c(SW, np.uint8)
    Bc, WLc = _c(B, np.uint16), _c(WL, np.uint16)
    S, N = QX.shape[0], QW.shape[0]
    H = SX.shape[1] * G
    KC = Bc.shape[1]
    assert WLc.shape == (N, KC)
    Y = np.zeros((S, N), np.float64)
    lib().orc_gemm_comp(_p(QX), _p(SX), afmt, _p(Bc), _p(QW), _p(SW), wfmt, _p(WLc), S, N, H, G, KC, _p(Y))
    return Y


def build_table_multi(Xcal: np.ndarray, G: int, m: int, alpha: float = 5.0, rho: float = 0.35):
    """-> (L int32[K, m], hits int32[K, m], events int32[K])."""
    Xcal = _c(Xcal, np.uint16)
    R, H = Xcal.shape
    K = H // G
    L = np.zeros((K, m), np.int32)
    hits = np.zeros((K, m), np.int32)
    events = np.zeros(K, np.int32)
    lib().orc_build_table_multi(_p(Xcal), R, H, G, float(alpha), float(rho), m, _p(L), _p(hits), _p(events))
    return L, hits, events


def osc_linear_multi(X, W, G: int, L, m: int):
    """The whole layer with m protected channels per group, in fp64."""
    QX, SX, B = quant_act_multi(X, G, L, m)
    QW, SW, WL = pack_weights_multi(W, G, L, m)
    return gemm_comp(QX, SX, QW, SW, G, B, WL)


# ------------------------------------------------ the MLP glue of a Qwen3-shaped block

def exp32(x: float) -> float:
    """The binary32 exponential the glue is defined with (Cody-Waite + Taylor, see osc_oracle.c)."""
    return float(lib().orc_exp32(float(x)))


def silu32(g: float) -> float:
    return float(lib().orc_silu32(float(g)))


def bf16_rne(f: float) -> int:
    return int(lib().orc_bf16_rne(float(f)))


def swiglu(GU: np.ndarray) -> np.ndarray:
    """GU: uint16 bf16 bits [S, 2F] (gate | up) -> h = bf16(silu(gate) * up), uint16 [S, F]."""
    GU = _c(GU, np.uint16)
    S, F2 = GU.shape
    assert F2 % 2 == 0
    F = F2 // 2
    Hh = np.zeros((S, F), np.uint16)
    lib().orc_swiglu(_p(GU), S, F, _p(Hh))
    return Hh


def swiglu_quant(GU: np.ndarray, G: int, L=None, m: int = 1, fmt: int = MXFP4):
    """The W2 input operand of the block: quantization (with extraction when L is given) of
    h = swiglu(GU).  -> (QX, SX, B or None)."""
    Hh = swiglu(GU)
    if L is None:
        return quant_act(Hh, G, None, fmt)
    return quant_act_multi(Hh, G, L, m, fmt)


def mean_density(hits: np.ndarray, events: np.ndarray) -> float:
    """§2.2 clustering density C averaged over the groups that saw an outlier event."""
    hits = _c(hits, np.int32)
    events = _c(events, np.int32)
    K = events.shape[0]
    m = hits.size // K
    return float(lib().orc_mean_density(_p(hits.reshape(K * m)), _p(events), K, m))


# ------------------------------------------------ G = 16 pairs in E3M2 (fast G = 16)

def e3m2_decode(code: int) -> float:
    return float(lib().orc_e3m2_decode(code))


def e3m2_encode(v: float) -> int:
    return int(lib().orc_e3m2_encode(float(v)))


def get_code6(Q6: np.ndarray, k: int) -> np.ndarray:
    """6-bit code k of every row of a packed E3M2 buffer (element k at bits [6k, 6k+6))."""
    bit = 6 * k
    b, sh = bit >> 3, bit & 7
    w = Q6[:, b].astype(np.uint32) >> sh
    if sh > 2:
        w |= Q6[:, b + 1].astype(np.uint32) << (8 - sh)
    return (w & 0x3F).astype(np.uint8)


def quant_act_fp6p(X: np.ndarray, L=None, m: int = 1):
    """G = 16 with extraction, re-encoded as E3M2 pairs -> (Q6 uint8[S, 3H/4], S32 uint8[S, H/32],
    B uint16[S, H/16*m] or None)."""
    X = _c(X, np.uint16)
    S, H = X.shape
    Q6 = np.zeros((S, 3 * H // 4), np.uint8)
    S32 = np.zeros((S, H // 32), np.uint8)
    B = None if L is None else np.zeros((S, H // 16 * m), np.uint16)
    Lc = None if L is None else _c(L, np.int32).reshape(-1)
    lib().orc_quant_act_fp6p(_p(X), S, H, _p(Lc), m, _p(Q6), _p(S32), _p(B))
    return Q6, S32, B


def pack_weights_fp6p(W: np.ndarray, L=None, m: int = 1):
    W = _c(W, np.uint16)
    N, H = W.shape
    Q6 = np.zeros((N, 3 * H // 4), np.uint8)
    S32 = np.zeros((N, H // 32), np.uint8)
    WL = None if L is None else np.zeros((N, H // 16 * m), np.uint16)
    Lc = None if L is None else _c(L, np.int32).reshape(-1)
    lib().orc_pack_weights_fp6p(_p(W), N, H, _p(Lc), m, _p(Q6), _p(S32), _p(WL))
    return Q6, S32, WL


def gemm_fp6p(Q6X, S32X, Q6W, S32W, B=None, WL=None) -> np.ndarray:
    """Y of E3M2-pair operands (scale blocks of 32) plus the compensation B WL^T (any width)."""
    Q6X, S32X, Q6W, S32W = (_c(a, np.uint8) for a in (Q6X, S32X, Q6W, S32W))
    S, N = Q6X.shape[0], Q6W.shape[0]
    H = S32X.shape[1] * 32
    Bc = None if B is None else _c(B, np.uint16)
    WLc = None if WL is None else _c(WL, np.uint16)
    KC = 0 if Bc is None else Bc.shape[1]
    Y = np.zeros((S, N), np.float64)
    lib().orc_gemm_comp(_p(Q6X), _p(S32X), FP6P, _p(Bc), _p(Q6W), _p(S32W), FP6P, _p(WLc), S, N, H, 32, KC, _p(Y))
    return Y
