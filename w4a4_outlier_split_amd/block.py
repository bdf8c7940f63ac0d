"""The linear layers of a Qwen3-8B-shaped transformer block run through libosc, each on the path
its input calls for (OSC page "W4A4量化技术：OSC框架如何实现高效LLM部署", §2.3 Table 1 and the
per-module rule that follows it, §4 for W2).

Host-side orchestration only: buffers are torch tensors (device memory), every step of every
layer runs in the library's kernels through the C ABI.  Attention itself (between QKV and Wo) and
the norms and residual adds are not part of this block: the Wo layer takes its input as given.

Per-module rule (§2.3): a module input's clustering density C is the share of a group's outlier
events captured by its statically indexed channel (§2.2), averaged over the groups that saw an
event; C >= 35 % keeps the 4-bit OSC path with the table, C < 35 % switches the module to FP8
microscaling activations (the §4 fallback; weights stay MXFP4 unless asked otherwise).  C is
measured on calibration rows of the module's own input; for the down-projection W2 those rows are
the glue output h = silu(gate) * up of the calibration rows pushed through the up-projection.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import (OSC_MAX_GROUPS, OSC_MXFP4, OSC_MXFP8, OSC_Y_BF16, code_bytes, osc_build_table_multi, osc_gemm_fp8,
               osc_gemm_multi, osc_pack_weights_multi, osc_quant_act_multi, osc_swiglu, osc_swiglu_quant,
               scale_bytes, side_elems)

DENSITY_THRESHOLD = 0.35  # §2.3: below it the module falls back to FP8 microscaling
ALPHA, RHO = 5.0, 0.35    # table-builder defaults (§3.1 / §5.2; rho: the 35 % line of §2.3)


def mean_density(hits: np.ndarray, events: np.ndarray) -> float:
    """§2.2's C averaged over the groups that saw an event (0 if none did); hits: the kept
    entry's count per group (first column when the table has m entries per group)."""
    hits = np.asarray(hits).reshape(len(events), -1)[:, 0].astype(np.float64)
    events = np.asarray(events).astype(np.float64)
    seen = events > 0
    return float(np.mean(hits[seen] / events[seen])) if seen.any() else 0.0


@dataclass
class Calibration:
    L: np.ndarray        # int32[K, m] table slice
    hits: np.ndarray     # int32[K, m]
    events: np.ndarray   # int32[K]
    density: float       # mean C over the groups with events
    path: str            # "osc" or "fp8"


def calibrate(torch, Xcal, H: int, G: int = 32, m: int = 1, stream=None,
              threshold: float = DENSITY_THRESHOLD) -> Calibration:
    """Build the table slice on the device from calibration rows Xcal [R, H] (bf16 device tensor)
    and apply the per-module rule."""
    R = Xcal.shape[0]
    K = H // G
    dev = Xcal.device
    L = torch.empty((K * m,), dtype=torch.int32, device=dev)
    hits = torch.empty((K * m,), dtype=torch.int32, device=dev)
    ev = torch.empty((K,), dtype=torch.int32, device=dev)
    osc_build_table_multi(Xcal, R, H, G, ALPHA, RHO, m, L, hits, ev, stream)
    torch.cuda.synchronize()
    Lh = L.cpu().numpy().reshape(K, m)
    hh = hits.cpu().numpy().reshape(K, m)
    eh = ev.cpu().numpy()
    c = mean_density(hh, eh)
    return Calibration(Lh, hh, eh, c, "osc" if c >= threshold else "fp8")


# ------------------------------------------------------------------ per-layer group size (§6)
# §6 names "dynamic group size" (G adapted per layer among 16 / 32 / 64) as a direction only.
# Reading: a larger G is faster (Table 2), but a group can protect only the channels its table
# entries list; G is too large for a layer when its groups often hold two persistent outlier
# channels.  For each candidate G, fastest first, the table is built with two entries per group on
# the layer's calibration rows; two_share = the share of the protected groups whose second entry
# is also kept (a second consistent channel).  The layer takes the largest G whose two_share is at
# most `tolerance`, else the G with the smallest two_share (larger G on ties).

GROUP_SIZES = (64, 32, 16)
TWO_SHARE_TOLERANCE = 0.10


def two_share(L2: np.ndarray) -> float:
    """L2: int[K, 2] table slice built with two entries per group."""
    L2 = np.asarray(L2).reshape(-1, 2)
    protected = L2[:, 0] >= 0
    if not protected.any():
        return 0.0
    return float(np.mean(L2[protected, 1] >= 0))


def choose_group_size(shares: dict, tolerance: float = TWO_SHARE_TOLERANCE) -> int:
    """shares: {G: two_share}.  The rule above."""
    for G in sorted(shares, reverse=True):
        if shares[G] <= tolerance:
            return G
    return min(sorted(shares, reverse=True), key=lambda g: shares[g])


def calibrate_group_size(torch, Xcal, H: int, sizes=GROUP_SIZES, tolerance: float = TWO_SHARE_TOLERANCE,
                         stream=None):
    """-> (chosen G, {G: two_share}) for one layer's calibration rows Xcal [R, H] (device bf16)."""
    shares = {}
    for G in sizes:
        if H % 256 == 0 and H // G * 2 <= OSC_MAX_GROUPS:
            shares[G] = two_share(calibrate(torch, Xcal, H, G, m=2, stream=stream).L)
    return choose_group_size(shares, tolerance), shares


class Linear:
    """One linear layer y = x W^T with W [N, H] bf16, packed once (offline, §3.3) for its path:
    "osc" (MXFP4 activations with the table's channels split off into B, MXFP4 weights and W_L)
    or "fp8" (MXFP8 activations, no split; weights in wfmt)."""

    def __init__(self, torch, W, N: int, H: int, G: int, path: str, L: Optional[np.ndarray] = None, m: int = 1,
                 wfmt: int = OSC_MXFP4, stream=None):
        if path not in ("osc", "fp8"):
            raise ValueError(f"unknown path {path!r}")
        if path == "osc" and L is None:
            raise ValueError("the OSC path needs a table slice")
        self.torch, self.N, self.H, self.G, self.path, self.m = torch, N, H, G, path, m
        self.L = None if path == "fp8" else np.ascontiguousarray(L, np.int32).reshape(H // G, m)
        self.afmt = OSC_MXFP4 if path == "osc" else OSC_MXFP8
        self.wfmt = OSC_MXFP4 if path == "osc" else wfmt
        dev = W.device
        u8 = lambda n: torch.empty((n,), dtype=torch.uint8, device=dev)
        self.QW, self.SW = u8(code_bytes(N, H, self.wfmt)), u8(scale_bytes(N, H, G))
        self.WL = (torch.empty((side_elems(N, H, G, m),), dtype=torch.int16, device=dev)
                   if self.L is not None else None)
        osc_pack_weights_multi(W, N, H, G, self.L, m, self.wfmt, self.QW, self.SW, self.WL, stream)

    def act_buffers(self, S: int, device):
        """Device buffers of the quantized activation operand for S rows."""
        t = self.torch
        QX = t.empty((code_bytes(S, self.H, self.afmt),), dtype=t.uint8, device=device)
        SX = t.empty((scale_bytes(S, self.H, self.G),), dtype=t.uint8, device=device)
        B = (t.empty((side_elems(S, self.H, self.G, self.m),), dtype=t.int16, device=device)
             if self.L is not None else None)
        return QX, SX, B

    def quantize(self, X, S: int, act, stream=None) -> None:
        QX, SX, B = act
        osc_quant_act_multi(X, S, self.H, self.G, self.L, self.m, self.afmt, QX, SX, B, stream)

    def gemm(self, act, S: int, Y, yt: int = OSC_Y_BF16, stream=None) -> None:
        QX, SX, B = act
        if self.path == "osc":
            osc_gemm_multi(QX, SX, B, self.QW, self.SW, self.WL, S, self.N, self.H, self.G, self.m, Y, yt, stream)
        else:
            osc_gemm_fp8(QX, SX, self.QW, self.SW, self.wfmt, S, self.N, self.H, self.G, Y, yt, stream)

    def forward(self, X, S: int, act, Y, yt: int = OSC_Y_BF16, stream=None) -> None:
        self.quantize(X, S, act, stream)
        self.gemm(act, S, Y, yt, stream)


class MLP:
    """Gated MLP: up-projection with W1 (gate) and W3 (up) stacked as one [2F, H] weight, the glue
    h = silu(gate) * up fused into the quantization of W2's input, then the down-projection W2
    [H, F]."""

    def __init__(self, up: Linear, down: Linear):
        if up.N != 2 * down.H:
            raise ValueError("the up-projection must produce [gate | up], twice W2's input width")
        self.up, self.down = up, down
        self.F = down.H

    def buffers(self, S: int, device):
        t = self.up.torch
        return {"x": self.up.act_buffers(S, device),
                "gu": t.empty((S, 2 * self.F), dtype=t.bfloat16, device=device),
                "h": self.down.act_buffers(S, device)}

    def forward(self, X, S: int, bufs, Y, yt: int = OSC_Y_BF16, stream=None) -> None:
        self.up.forward(X, S, bufs["x"], bufs["gu"], OSC_Y_BF16, stream)
        QX, SX, B = bufs["h"]
        d = self.down
        osc_swiglu_quant(bufs["gu"], S, self.F, d.G, d.L, d.m, d.afmt, QX, SX, B, stream)
        d.gemm(bufs["h"], S, Y, yt, stream)

    def glue_rows(self, torch, Xcal, stream=None):
        """W2's calibration rows: Xcal [R, H] pushed through the up-projection and the glue."""
        R = Xcal.shape[0]
        dev = Xcal.device
        act = self.up.act_buffers(R, dev)
        gu = torch.empty((R, 2 * self.F), dtype=torch.bfloat16, device=dev)
        self.up.forward(Xcal, R, act, gu, OSC_Y_BF16, stream)
        h = torch.empty((R, self.F), dtype=torch.bfloat16, device=dev)
        osc_swiglu(gu, R, self.F, h, stream)
        return h

    def calibrate_down(self, torch, Xcal, G: int = 32, m: int = 1, stream=None,
                       threshold: float = DENSITY_THRESHOLD) -> Calibration:
        """The per-module rule on W2's calibration rows (glue_rows)."""
        return calibrate(torch, self.glue_rows(torch, Xcal, stream), self.F, G, m, stream, threshold)
