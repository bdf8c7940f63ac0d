"""Exact-rational restatement of the OSC W4A4 layer, for pinning the oracle on tiny inputs.

Written independently of ``oracle/`` (no shared code): every value is a
``fractions.Fraction``, element grids are spelled out from the OCP MX v1.0
format definitions, rounding is "nearest, ties to the even grid index" by
exact comparison, and the shared exponent is found by searching for the
integer e with 2^(e+emax) <= amax < 2^(e+emax+1).

Follows the OSC page ("W4A4量化技术：OSC框架如何实现高效LLM部署"): §3.2 (zero and
extract the indexed channel into B, scale the zeroed group, dual-path output
Y = (Q_X ⊗ Q_W)·S + B·W_L) and §4 (FP8 microscaling, no extraction).
"""
from fractions import Fraction as F
from typing import List, Optional, Sequence

# OCP MX v1.0, FP4 E2M1 magnitudes in code order 0..7.
E2M1_GRID = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def _e4m3_grid() -> List[F]:
    g = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue  # NaN
            g.append(F(m, 8) * F(1, 64) if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7))
    return g


E4M3_GRID = _e4m3_grid()  # 127 magnitudes, code order 0..126, max 448


def bf16(bits: int) -> F:
    s = -1 if (bits >> 15) & 1 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF, "non-finite input"
    if e == 0:
        return s * F(m, 128) * F(2) ** -126
    return s * (1 + F(m, 128)) * F(2) ** (e - 127)


def is_negative(bits: int) -> bool:
    return bool((bits >> 15) & 1)


def round_grid(v: F, grid: Sequence[F]) -> int:
    """Index of the nearest magnitude of |v| in grid (ties -> even index); saturating."""
    m = abs(v)
    if m >= grid[-1]:
        return len(grid) - 1
    best, bestd = 0, None
    for i, g in enumerate(grid):
        d = abs(m - g)
        if bestd is None or d < bestd or (d == bestd and i % 2 == 0):
            best, bestd = i, d
    return best


def shared_exp(amax: F, emax: int) -> int:
    if amax == 0:
        return -127
    e = 0
    while F(2) ** (e + emax) > amax:
        e -= 1
    while F(2) ** (e + emax + 1) <= amax:
        e += 1
    return max(-127, min(127, e))


def quant_group(vals: List[F], neg: List[bool], fp8: bool):
    grid = E4M3_GRID if fp8 else E2M1_GRID
    sign_bit = 0x80 if fp8 else 0x8
    amax = max(abs(v) for v in vals)
    e = shared_exp(amax, 8 if fp8 else 2)
    codes = []
    for v, n in zip(vals, neg):
        idx = round_grid(v / F(2) ** e, grid)
        codes.append((sign_bit if n else 0) | idx)
    return e, codes


def decode(code: int, fp8: bool) -> F:
    if fp8:
        mag = E4M3_GRID[code & 0x7F]
        return -mag if code & 0x80 else mag
    mag = E2M1_GRID[code & 7]
    return -mag if code & 8 else mag


def _channels(entry) -> List[int]:
    """A table entry: one offset (the page's single channel) or a sequence of them (§6)."""
    return list(entry) if isinstance(entry, (list, tuple)) else [entry]


def quant_rows(rows: List[List[int]], G: int, L: Optional[List], fp8: bool):
    """rows: bf16 bit patterns.  Returns (codes[s][h], exps[s][k], B[s][c] bf16 bits).
    L[k] is an offset (-1 = none) or a list of m of them; B then has one column per listed
    entry, group-major (column k*m + j)."""
    codes_all, exps_all, b_all = [], [], []
    for row in rows:
        H = len(row)
        codes_row, exps_row, b_row = [], [], []
        for k in range(H // G):
            bits = list(row[k * G:(k + 1) * G])
            vals = [bf16(b) for b in bits]
            neg = [is_negative(b) for b in bits]
            if L is not None:
                chans = _channels(L[k])
                for c in chans:
                    b_row.append(bits[c] if c >= 0 else 0)
                for c in chans:
                    if c >= 0:
                        vals[c] = F(0)
                        neg[c] = False
            e, codes = quant_group(vals, neg, fp8)
            codes_row += codes
            exps_row.append(e)
        codes_all.append(codes_row)
        exps_all.append(exps_row)
        b_all.append(b_row)
    return codes_all, exps_all, b_all


def osc_linear(X: List[List[int]], W: List[List[int]], G: int, L: Optional[List[int]], act_fp8: bool = False,
               w_fp8: bool = False) -> List[List[F]]:
    """Exact Y[s][n] of the whole layer: quantize X (with extraction unless act_fp8), quantize W,
    dual-path product."""
    Lx = None if act_fp8 else L
    qx, ex, bx = quant_rows(X, G, Lx, act_fp8)
    qw, ew, _ = quant_rows(W, G, None, w_fp8)
    H = len(X[0])
    K = H // G
    Y = []
    for s in range(len(X)):
        out = []
        for n in range(len(W)):
            y = F(0)
            for k in range(K):
                part = sum(decode(qx[s][k * G + j], act_fp8) * decode(qw[n][k * G + j], w_fp8) for j in range(G))
                y += part * F(2) ** (ex[s][k] + ew[n][k])
            if Lx is not None:
                col = 0
                for k in range(K):
                    for c in _channels(L[k]):
                        if c >= 0:
                            y += bf16(bx[s][col]) * bf16(W[n][k * G + c])
                        col += 1
            out.append(y)
        Y.append(out)
    return Y
