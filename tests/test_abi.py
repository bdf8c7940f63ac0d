"""C-ABI checks that need no GPU: libosc loads, exports every function include/osc.h declares,
and rejects invalid arguments with the documented status before any HIP call (so no
kernel is launched and no pointer is dereferenced; the fake addresses below are never
touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "osc.h")

osc = pytest.importorskip("w4a4_outlier_split_amd", reason="libosc.so not built")

A = 0x10000  # 16-byte aligned fake device address (never dereferenced by a rejected call)
U = 0x10008  # misaligned


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:osc_status|const char\*)\s+(osc_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(osc.EXPORTS)
    lib = ctypes.CDLL(osc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in osc.STATUS.items():
        assert osc.osc_status_str(code).startswith(name)


def status(fn, *args):
    r = getattr(osc._lib, fn)(*args)
    return r


def L8(vals):
    arr = np.asarray(vals, np.int32)
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def test_quant_act_validation():
    keep, lp = L8([-1] * 8)
    q = lambda X=A, S=16, H=256, G=32, l=lp, f=0, QX=A, SX=A, B=A: status("osc_quant_act", X, S, H, G, l, f, QX, SX, B, None)
    assert q(f=7) == 5                      # bad format
    assert q(G=8) == 2 and q(G=128) == 2     # G not in {16, 32, 64}
    assert q(H=250) == 2                     # H % G != 0
    assert q(H=384) == 2                     # tiled layout: H % 256 != 0
    assert q(S=1 << 22, H=4096) == 2         # S * H >= 2^34
    assert q(S=1 << 24, H=256) == 2          # S >= 2^24 (32-bit panel offsets)
    assert q(S=(1 << 24) - 1, H=256, X=U) == 4  # the largest S passes the shape checks
    assert q(S=-1) == 2
    assert q(X=None) == 1 and q(QX=None) == 1 and q(SX=None) == 1
    assert q(B=None) == 1                    # table given but no B
    assert q(l=None) == 1                    # B given but no table
    assert q(X=U) == 4 and q(B=U) == 4
    bad, bp = L8([0, 1, 2, 32, -1, -1, -1, -1])
    assert q(l=bp) == 3                      # entry >= G
    bad2, bp2 = L8([0, -2, 0, 0, 0, 0, 0, 0])
    assert q(l=bp2) == 3
    assert q(H=1024 * 64 + 64, G=64, l=None, B=None) == 2  # K > OSC_MAX_GROUPS


def test_pack_weights_validation():
    keep, lp = L8([3] * 8)
    p = lambda W=A, N=128, H=256, G=32, l=lp, f=0, QW=A, SW=A, WL=A: status("osc_pack_weights", W, N, H, G, l, f, QW, SW, WL, None)
    assert p(f=2) == 5
    assert p(WL=None) == 1 and p(l=None) == 1
    assert p(W=U) == 4 and p(SW=U) == 4
    assert p(N=-3) == 2
    assert p(H=384) == 2
    assert p(N=1 << 24) == 2
    bad, bp = L8([3, 3, 3, 3, 3, 3, 3, 40])
    assert p(l=bp) == 3


def test_fp8_fallback_refuses_a_table():
    """The FP8 fallback (§4) extracts nothing and osc_gemm_fp8 takes no B / W_L: a table with
    OSC_MXFP8 would zero channels that no later call adds back, so it is refused up front."""
    keep, lp = L8([-1] * 8)  # even an all -1 table: the combination itself is refused
    two, tp = L8([0, 5] * 8)
    qa = lambda l, B, m=1: status("osc_quant_act_multi", A, 16, 256, 32, l, m, 1, A, A, B, None)
    assert qa(lp, A) == 5 and qa(tp, A, m=2) == 5
    assert status("osc_quant_act", A, 16, 256, 32, lp, 1, A, A, A, None) == 5
    assert status("osc_quant_act", A, 0, 256, 32, lp, 1, A, A, A, None) == 5  # even with nothing to do
    pw = lambda l, WL, m=1: status("osc_pack_weights_multi", A, 64, 256, 32, l, m, 1, A, A, WL, None)
    assert pw(lp, A) == 5 and pw(tp, A, m=2) == 5
    assert status("osc_pack_weights", A, 64, 256, 32, lp, 1, A, A, A, None) == 5
    # the same formats without a table are valid up to the pointer checks
    assert status("osc_quant_act", U, 16, 256, 32, None, 1, A, A, None, None) == 4
    assert status("osc_pack_weights", U, 64, 256, 32, None, 1, A, A, None, None) == 4


def test_gemm_validation():
    g = lambda QX=A, SX=A, B=A, QW=A, SW=A, WL=A, S=16, N=128, H=256, G=32, Y=A, yt=0: status(
        "osc_gemm", QX, SX, B, QW, SW, WL, S, N, H, G, Y, yt, None)
    assert g(yt=3) == 5
    assert g(H=384) == 2                     # H % 256 != 0
    assert g(H=256, G=64) == 2               # K = 4: compensation needs K % 8 == 0
    assert g(B=None) == 1 and g(WL=None) == 1
    assert g(Y=None) == 1
    assert g(Y=U) == 4 and g(WL=U) == 4
    assert g(S=-1) == 2 and g(N=-1) == 2
    assert g(S=0) == 0 and g(N=0) == 0       # valid, nothing launched
    assert g(S=1 << 24) == 2 and g(N=1 << 24) == 2          # rows >= 2^24
    assert g(S=1 << 22, H=4096) == 2 and g(N=1 << 22, H=4096) == 2  # rows * H >= 2^34


def test_gemm_fp8_validation():
    f = lambda QX=A, SX=A, QW=A, SW=A, wf=0, S=16, N=128, H=256, G=32, Y=A, yt=0: status(
        "osc_gemm_fp8", QX, SX, QW, SW, wf, S, N, H, G, Y, yt, None)
    assert f(wf=9) == 5
    assert f(G=16) == 2
    assert f(QW=None) == 1
    assert f(SX=U) == 4
    assert f(S=0) == 0


def test_build_table_validation():
    b = lambda X=A, R=1536, H=256, G=32, al=5.0, rho=0.35, L=A, hi=A, ev=A: status(
        "osc_build_table", X, R, H, G, ctypes.c_double(al), ctypes.c_double(rho), L, hi, ev, None)
    assert b(R=0) == 2
    assert b(al=0.0) == 2 and b(rho=0.0) == 2 and b(rho=1.5) == 2
    assert b(L=None) == 1
    assert b(X=U) == 4


def test_multi_validation():
    K = 8  # H=256, G=32
    good, gp = L8([0, 5] * K)
    dup, dp = L8([3, 3] + [0, 5] * (K - 1))        # channel listed twice in group 0
    q = lambda l=gp, m=2, H=256, B=A: status("osc_quant_act_multi", A, 16, H, 32, l, m, 0, A, A, B, None)
    assert q(m=0) == 2 and q(m=4) == 2           # 1 <= m <= OSC_MAX_CHANNELS
    assert q(l=dp) == 3                           # duplicate channel in a group
    bad, bp = L8([0, 32] * K)
    assert q(l=bp) == 3                           # entry >= G
    none_ok, np_ = L8([-1, -1] * K)
    assert q(l=np_, H=384) == 2                   # tiled layout: H % 256
    p = lambda l=gp, m=2: status("osc_pack_weights_multi", A, 64, 256, 32, l, m, 0, A, A, A, None)
    assert p(l=dp) == 3 and p(m=5) == 2
    g = lambda m=2, H=256, G=32, B=A, WL=A: status("osc_gemm_multi", A, A, B, A, A, WL, 16, 64, H, G, m, A, 0, None)
    assert g(m=0) == 2
    assert g(H=256, G=64, m=1) == 2               # compensation columns m*K = 4: not a multiple of 8
    assert g(H=256, G=64, m=3) == 2               # 12 columns
    assert g(H=65536, G=64, m=2) == 2             # m*K = 2048 > OSC_MAX_GROUPS
    b = lambda m=2: status("osc_build_table_multi", A, 1536, 256, 32, ctypes.c_double(5.0), ctypes.c_double(0.35),
                           m, A, A, A, None)
    assert b(m=0) == 2 and b(m=4) == 2


def test_swiglu_quant_validation():
    keep, lp = L8([-1] * 16)  # F=512, G=32: K=16
    q = lambda GU=A, S=16, F=512, G=32, l=lp, m=1, f=0, QX=A, SX=A, B=A: status(
        "osc_swiglu_quant", GU, S, F, G, l, m, f, QX, SX, B, None)
    assert q(f=5) == 5                       # bad format
    assert q(f=1) == 5 and q(f=1, m=2, l=L8([-1] * 32)[1]) == 5  # FP8 fallback with a table
    assert q(f=1, l=None, B=None, GU=U) == 4  # FP8 without a table passes the format check
    assert q(F=384) == 2                     # tiled layout: F % 256
    assert q(G=8) == 2
    assert q(m=0) == 2 and q(m=4) == 2
    assert q(S=1 << 24) == 2                 # rows >= 2^24
    assert q(S=(1 << 21) + 8, F=4096) == 2   # S * 2F >= 2^34 (S * F alone is below)
    assert q(GU=None) == 1 and q(SX=None) == 1
    assert q(B=None) == 1 and q(l=None) == 1  # table and B go together
    assert q(GU=U) == 4 and q(QX=U) == 4
    bad, bp = L8([0] * 15 + [32])
    assert q(l=bp) == 3
    assert q(S=0) == 0                       # nothing to do


def test_swiglu_validation():
    h = lambda GU=A, S=16, F=512, Ho=A: status("osc_swiglu", GU, S, F, Ho, None)
    assert h(F=12) == 2 and h(F=0) == 2 and h(S=-1) == 2
    assert h(S=1 << 24) == 2
    assert h(GU=None) == 1 and h(Ho=None) == 1
    assert h(GU=U) == 4 and h(Ho=U) == 4
    assert h(S=0) == 0


def test_linear_decode_validation():
    keep, lp = L8([-1] * 8)  # H=256, G=32: K=8
    d = lambda X=A, S=16, H=256, G=32, l=lp, m=1, QW=A, SW=A, WL=A, N=128, Y=A, yt=0: status(
        "osc_linear_decode", X, S, H, G, l, m, QW, SW, WL, N, Y, yt, None)
    assert d(S=33) == 2                      # decode sizes only
    assert d(S=-1) == 2 and d(N=-1) == 2
    assert d(yt=2) == 5
    assert d(H=384) == 2
    assert d(m=4) == 2
    assert d(H=256, G=64, l=L8([-1] * 4)[1]) == 2  # compensation columns 4: not a multiple of 8
    assert d(H=16384, G=32, l=None, WL=None) == 2  # 256 KiB of quantized rows: more than LDS holds
    assert d(WL=None) == 1 and d(l=None) == 1
    assert d(X=None) == 1 and d(Y=None) == 1
    assert d(X=U) == 4 and d(WL=U) == 4
    bad, bp = L8([0, 1, 2, 3, 4, 5, 6, 40])
    assert d(l=bp) == 3
    assert d(S=0) == 0 and d(N=0) == 0


def test_fp6p_validation():
    keep, lp = L8([-1] * 16)  # H=256, G=16: K=16
    q = lambda G=16, f=2, l=lp, B=A: status("osc_quant_act_multi", A, 16, 256, G, l, 1, f, A, A, B, None)
    assert q(G=32, l=L8([-1] * 8)[1]) == 5    # E3M2 pairs exist for G = 16 only
    p = lambda G=16, f=2: status("osc_pack_weights_multi", A, 64, 256, G, None, 1, f, A, A, None, None)
    assert p(G=64) == 5
    g = lambda S=16, N=64, H=256, m=1, B=A, WL=A, yt=0: status("osc_gemm_fp6p", A, A, B, A, A, WL, S, N, H, m, A, yt,
                                                                None)
    assert g(H=384) == 2 and g(m=0) == 2 and g(yt=4) == 5
    assert g(B=None) == 1
    assert g(S=0) == 0
    assert g(H=256 * 64 + 256) == 2          # H/16 > OSC_MAX_GROUPS
