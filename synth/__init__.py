"""Seeded synthetic inputs for the OSC W4A4 linear layer.

This module is shared by the tests, the benchmark and the oracle-side checks,
and it deliberately holds none of the method's arithmetic: it only draws
activations, weights and calibration rows with the structure the OSC write-up
describes (page "W4A4量化技术：OSC框架如何实现高效LLM部署", §2.1: high-magnitude
outliers that stay in fixed channels on every token, "vertical stripes";
§2.3 / Table 1: the share of such groups differs by module input; §5.2:
3 x 512 calibration tokens).  The pages measure on Qwen3-8B activations and
the Pile; neither is available, so these seeded draws stand in for them.

Every array is returned as raw bf16 bit patterns (``numpy.uint16``).  fp32
draws are rounded to bf16 by PyTorch's round-to-nearest-even conversion.

Recipe (one ``numpy.random.default_rng(seed)`` per role, PCG64):
  * plant:  choose ``round(frac*K32)`` groups of 32 channels without
    replacement, then per chosen group an offset in [0, 32) and a factor
    ``uniform(lo, hi)``, drawn group by group in the chosen order;
  * z:      base draws, ``standard_normal`` (or ``laplace(0, 1)``) of shape S x H;
  * x = z, then every token's planted channel is multiplied by its factor;
  * spikes: an independent Bernoulli(p) mask per element multiplies by 20
    (QKV-style inputs), or one x20 spike per token at a uniformly random
    channel of every unplanted group (down-projection-style inputs);
  * W:      ``standard_normal(N, H) * 0.02``.
Calibration rows reuse the plant but draw fresh z and spikes from their own
seeds.  A smaller S is the row prefix of a larger S from the same seeds.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

PLANT_BLOCK = 32  # outliers are planted per 32-channel block (the G=32 grouping)
CALIB_ROWS = 3 * 512


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32/fp64 array -> bf16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Plant:
    groups: np.ndarray    # int64[n] 32-channel block indices
    offsets: np.ndarray   # int64[n] offset of the persistent channel in its block
    factors: np.ndarray   # float64[n]

    @property
    def channels(self) -> np.ndarray:
        return self.groups * PLANT_BLOCK + self.offsets


def draw_plant(seed: int, H: int, frac: float, lo: float, hi: float, count: Optional[int] = None) -> Plant:
    rng = np.random.default_rng(seed)
    nblk = H // PLANT_BLOCK
    n = int(round(frac * nblk)) if count is None else count
    groups = rng.choice(nblk, n, replace=False)
    offsets = np.empty(n, dtype=np.int64)
    factors = np.empty(n, dtype=np.float64)
    for i in range(n):
        offsets[i] = rng.integers(0, PLANT_BLOCK)
        factors[i] = rng.uniform(lo, hi)
    return Plant(groups.astype(np.int64), offsets, factors)


def _apply_plant(x: np.ndarray, plant: Plant) -> None:
    x[:, plant.channels] *= plant.factors.astype(np.float32)[None, :]


def draw_x_bernoulli_spikes(S: int, H: int, plant: Plant, seed_z: int, seed_spike: Optional[int],
                            p: float = 1e-3, spike: float = 20.0) -> np.ndarray:
    z = np.random.default_rng(seed_z).standard_normal((S, H), dtype=np.float32)
    _apply_plant(z, plant)
    if seed_spike is not None:
        mask = np.random.default_rng(seed_spike).random((S, H), dtype=np.float32) < p
        z[mask] *= spike
    return to_bf16_bits(z)


def draw_x_laplace_group_spikes(S: int, H: int, plant: Plant, seed_z: int, seed_spike: int,
                                spike: float = 20.0) -> np.ndarray:
    z = np.random.default_rng(seed_z).laplace(0.0, 1.0, (S, H)).astype(np.float32)
    _apply_plant(z, plant)
    nblk = H // PLANT_BLOCK
    free = np.setdiff1d(np.arange(nblk), plant.groups)
    offs = np.random.default_rng(seed_spike).integers(0, PLANT_BLOCK, (S, free.size))
    cols = free[None, :] * PLANT_BLOCK + offs
    rows = np.repeat(np.arange(S)[:, None], free.size, axis=1)
    z[rows, cols] *= spike
    return to_bf16_bits(z)


def draw_x_normal_group_spikes(S: int, H: int, plant: Plant, seed_z: int, seed_spike: int,
                               spike: float = 20.0) -> np.ndarray:
    """As draw_x_laplace_group_spikes with standard-normal base draws."""
    z = np.random.default_rng(seed_z).standard_normal((S, H), dtype=np.float32)
    _apply_plant(z, plant)
    nblk = H // PLANT_BLOCK
    free = np.setdiff1d(np.arange(nblk), plant.groups)
    offs = np.random.default_rng(seed_spike).integers(0, PLANT_BLOCK, (S, free.size))
    cols = free[None, :] * PLANT_BLOCK + offs
    rows = np.repeat(np.arange(S)[:, None], free.size, axis=1)
    z[rows, cols] *= spike
    return to_bf16_bits(z)


def draw_w(N: int, H: int, seed: int, std: float = 0.02) -> np.ndarray:
    w = np.random.default_rng(seed).standard_normal((N, H), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(w)


def planted_table(plant: Plant, H: int, G: int) -> np.ndarray:
    """The planted channels expressed as a table slice at group size G (-1 = none).

    Used only where the workload itself defines L as the planted channels (the
    tiny case).  If two planted channels fall into one G-group, the first in
    channel order is kept.
    """
    K = H // G
    L = np.full(K, -1, dtype=np.int32)
    for c in sorted(plant.channels.tolist()):
        k = c // G
        if L[k] < 0:
            L[k] = c - k * G
    return L


@dataclasses.dataclass
class Workload:
    name: str
    S: int
    H: int
    N: int
    G: int
    X: np.ndarray                      # uint16[S, H] bf16 bits
    w_seed: int                        # W (uint16[N, H] bf16 bits) is drawn on first access
    calib: Optional[np.ndarray] = None  # uint16[1536, H] bf16 bits, for the table builder
    L: Optional[np.ndarray] = None      # int32[K] when the workload fixes the table itself
    plant: Optional[Plant] = None
    _w: Optional[np.ndarray] = None

    @property
    def W(self) -> np.ndarray:
        if self._w is None:
            self._w = draw_w(self.N, self.H, self.w_seed)
        return self._w


def tiny() -> Workload:
    """S=16, H=256, N=128, G=32: 6 of 8 groups carry a x64 persistent channel; L = those channels."""
    S, H, N, G = 16, 256, 128, 32
    plant = draw_plant(1, H, 0.0, 64.0, 64.0, count=6)
    X = draw_x_bernoulli_spikes(S, H, plant, seed_z=2, seed_spike=None)
    return Workload("tiny", S, H, N, G, X, 4, None, planted_table(plant, H, G), plant)


def qkv(S: int = 2048, G: int = 32, seed_x: int = 12, seed_spike: int = 13) -> Workload:
    """Qwen3-8B QKV projection: H=4096, N=6144; 70% of groups x U(40,100); 0.1% x20 spikes."""
    H, N = 4096, 6144
    plant = draw_plant(11, H, 0.70, 40.0, 100.0)
    X = draw_x_bernoulli_spikes(S, H, plant, seed_x, seed_spike)
    calib = draw_x_bernoulli_spikes(CALIB_ROWS, H, plant, 14, 14 + 100)
    return Workload(f"qkv_s{S}_g{G}", S, H, N, G, X, 15, calib, None, plant)


def ffn_up(S: int = 4096) -> Workload:
    """Qwen3-8B FFN up/gate (W1 and W3 stacked): H=4096, N=24576; 65% of groups x U(30,80)."""
    H, N, G = 4096, 2 * 12288, 32
    plant = draw_plant(21, H, 0.65, 30.0, 80.0)
    X = draw_x_bernoulli_spikes(S, H, plant, 22, None)
    calib = draw_x_bernoulli_spikes(CALIB_ROWS, H, plant, 24, None)
    return Workload(f"ffn_up_s{S}", S, H, N, G, X, 25, calib, None, plant)


def ffn_down(S: int = 4096) -> Workload:
    """Qwen3-8B down-projection W2: H=12288, N=4096; Laplace(0,1); 25% persistent groups,
    the rest one x20 spike per token at a random channel."""
    H, N, G = 12288, 4096, 32
    plant = draw_plant(31, H, 0.25, 40.0, 100.0)
    X = draw_x_laplace_group_spikes(S, H, plant, 32, 33)
    calib = draw_x_laplace_group_spikes(CALIB_ROWS, H, plant, 34, 34 + 100)
    return Workload(f"ffn_down_s{S}", S, H, N, G, X, 35, calib, None, plant)


def attn_out(S: int = 4096) -> Workload:
    """Qwen3-8B attention output projection Wo: H=N=4096; N(0,1); 45% of groups x U(40,100)
    persistent, every other group one x20 spike per token at a random channel (Table 1 puts
    this input's clustering density at 40-50 %)."""
    H, N, G = 4096, 4096, 32
    plant = draw_plant(61, H, 0.45, 40.0, 100.0)
    X = draw_x_normal_group_spikes(S, H, plant, 62, 63)
    calib = draw_x_normal_group_spikes(CALIB_ROWS, H, plant, 64, 64 + 100)
    return Workload(f"attn_out_s{S}", S, H, N, G, X, 65, calib, None, plant)


def group_sweep(S: int, G: int) -> Workload:
    """QKV shape with the QKV plant and weights, X from its own seeds, any G in {16, 32, 64}."""
    w = qkv(S=S, G=G, seed_x=42, seed_spike=43)
    w.name = f"gsweep_s{S}_g{G}"
    return w


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) bf16 bits, for small edge-case tests."""
    z = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return to_bf16_bits(z)


def draw_plant_pairs(seed: int, H: int, frac_pair: float, frac_single: float, lo: float, hi: float) -> Plant:
    """Plant two persistent channels in round(frac_pair*K32) blocks and one in
    round(frac_single*K32) other blocks; offsets inside a pair are distinct."""
    rng = np.random.default_rng(seed)
    nblk = H // PLANT_BLOCK
    n2, n1 = int(round(frac_pair * nblk)), int(round(frac_single * nblk))
    blocks = rng.choice(nblk, n2 + n1, replace=False)
    groups, offsets, factors = [], [], []
    for i, b in enumerate(blocks):
        offs = rng.choice(PLANT_BLOCK, 2 if i < n2 else 1, replace=False)
        for o in offs:
            groups.append(b)
            offsets.append(o)
            factors.append(rng.uniform(lo, hi))
    return Plant(np.array(groups, np.int64), np.array(offsets, np.int64), np.array(factors))


def planted_table_multi(plant: Plant, H: int, G: int, m: int) -> np.ndarray:
    """The planted channels as an m-entry table slice (offsets ascending, -1 padded)."""
    K = H // G
    L = np.full((K, m), -1, dtype=np.int32)
    per = {}
    for c in plant.channels.tolist():
        per.setdefault(c // G, []).append(c % G)
    for k, offs in per.items():
        offs = sorted(offs)[:m]
        L[k, :len(offs)] = offs
    return L


def two_outlier_groups(S: int = 2048) -> Workload:
    """QKV shape (H=4096, N=6144, G=32) where 40% of the groups carry two persistent channels
    (x U(40,100) each) and 30% carry one; 0.1% x20 spikes.  L = the planted channels, 2 per group
    (the page's §6 case for protecting more than one channel)."""
    H, N, G = 4096, 6144, 32
    plant = draw_plant_pairs(51, H, 0.40, 0.30, 40.0, 100.0)
    X = draw_x_bernoulli_spikes(S, H, plant, 52, 53)
    calib = draw_x_bernoulli_spikes(CALIB_ROWS, H, plant, 54, 54 + 100)
    return Workload(f"two_outlier_s{S}", S, H, N, G, X, 55, calib, planted_table_multi(plant, H, G, 2), plant)

