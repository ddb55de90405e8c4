"""Seeded synthetic inputs and the named workloads (shared by both sides).

This module holds no arithmetic of the attention method: it only describes
problem shapes and draws Q/K/V.  The GPU path and the CPU oracle both take
their inputs from here, so the same bits reach both.

Workloads follow the shapes of the BASA pages' benchmarks (paperlayer.ai
summary of arXiv 2610.08772v1, sec. 4.1 and A.2: FLUX.1-dev image
extrapolation to 2048x2048 and Wan2.1 video extrapolation).  No dataset,
prompt or trained weight is used: activations are synthetic.

Recipe (per workload seed):
* Q, K, V ~ N(0, 1) i.i.d., drawn as float32 in [B, H, N, d] order from
  numpy's Philox generator keyed by (seed, stream) with streams Q=0, K=1, V=2;
* optionally a smooth low-rank component (stream 3) added to both Q and K:
  alpha * sum_r phi_r(t, y, x) * u_r^(h), with R = 4, alpha = 0.35,
  phi_r = cos(2 pi (a_r y / H + b_r x / W + c_r t / T) + theta_r),
  a_r, b_r in {0..3} not both zero, c_r in {0, 1, 2} (0 for images),
  theta_r ~ U[0, 2 pi), u_r^(h) ~ N(0, I_d) per head -- nearby tokens then
  get aligned logits, so the window router has real structure to find;
* bf16 workloads round every value to bfloat16 with round-to-nearest-even;
  the oracle receives exactly those values widened to float32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]
    window: Tuple[int, int, int]
    shift: Tuple[int, int, int]          # shift of the odd blocks; even blocks use 0
    pool: Tuple[int, int, int]
    topk: int
    dtype: str                           # "bf16" or "f32"
    seed: int
    smooth: bool
    description: str
    radius: int = -1                     # routing candidate radius (-1: every window)
    text: int = 0                        # extra global K/V rows (text tokens)

    @property
    def n_tokens(self) -> int:
        return int(np.prod(self.grid))


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, 1, 64, (1, 32, 32), (1, 8, 8), (0, 4, 4), (1, 4, 4), 0, "f32", 0,
                 False, "32x32 grid, 1 head, d=64, fp32, 8x8 windows, shift (4,4), 4x4 pool"),
        Workload("flux1k", 1, 24, 128, (1, 64, 64), (1, 16, 16), (0, 8, 8), (1, 4, 4), 0, "bf16",
                 1, False, "FLUX-shaped 1024x1024: 64x64 grid, 24 heads, d=128, 16x16 windows, "
                 "shift (8,8), 4x4 pool"),
        Workload("flux2k", 1, 24, 128, (1, 128, 128), (1, 32, 32), (0, 16, 16), (1, 8, 8), 0,
                 "bf16", 2, False, "FLUX-shaped 2048x2048: 128x128 grid, 24 heads, d=128, "
                 "32x32 windows, shift (16,16), 8x8 pool"),
        Workload("flux4k", 1, 24, 128, (1, 256, 256), (1, 32, 32), (0, 16, 16), (1, 16, 16), 0,
                 "bf16", 3, True, "FLUX-shaped 4096x4096: 256x256 grid, 24 heads, d=128, "
                 "32x32 windows, shift (16,16), 16x16 pool, smooth low-rank Q/K"),
        Workload("wan", 1, 12, 128, (21, 30, 52), (3, 10, 13), (1, 5, 6), (3, 5, 4), 4, "bf16",
                 4, True, "Wan-shaped video: 21x30x52 grid, 12 heads, d=128, 3x10x13 windows, "
                 "shift (1,5,6), 3x5x4 pool, top-4 routed windows, smooth low-rank Q/K"),
        Workload("wan_t3", 1, 12, 128, (21, 60, 104), (21, 15, 26), (0, 7, 13), (1, 4, 4), 1,
                 "bf16", 5, True, "Wan2.1 1664x960 video at the pages' Table 3 shape: 21x60x104 "
                 "grid, 12 heads, d=128, 15x26 spatial windows over all 21 frames, shift "
                 "(0,7,13), spatial 4x4 pool, one routed window within radius 1, smooth "
                 "low-rank Q/K", radius=1),
        Workload("wan_t3w10", 1, 12, 128, (21, 60, 104), (21, 10, 10), (0, 5, 5), (1, 4, 4), 1,
                 "bf16", 6, True, "Wan2.1 1664x960 video at Table 3's 10x10-window shape: "
                 "21x60x104 grid, 12 heads, d=128, 10x10 spatial windows over all 21 frames "
                 "(the last window column 4 wide: 104 = 10*10 + 4), shift (0,5,5), spatial 4x4 "
                 "pool, one routed window within radius 1, smooth low-rank Q/K", radius=1),
        Workload("flux2k_text", 1, 24, 128, (1, 128, 128), (1, 32, 32), (0, 16, 16), (1, 8, 8),
                 0, "bf16", 7, False, "FLUX-shaped 2048x2048 with its 512 text tokens as extra "
                 "global K/V rows: 128x128 grid, 24 heads, d=128, 32x32 windows, shift (16,16), "
                 "8x8 pool", text=512),
    ]
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=np.array([seed, stream], dtype=np.uint64)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exact float32 values."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def _smooth(w: Workload, rng: np.random.Generator, alpha: float = 0.35, rank: int = 4):
    T, H, W = w.grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    phis = []
    for _ in range(rank):
        while True:
            a, b = rng.integers(0, 4, size=2)
            if a or b:
                break
        c = int(rng.integers(0, 3)) if T > 1 else 0
        theta = rng.uniform(0.0, 2.0 * np.pi)
        phi = np.cos(2 * np.pi * (a * y / H + b * x / W + c * t / T) + theta)
        phis.append(phi.reshape(-1).astype(np.float32))
    phi = np.stack(phis, axis=1)                                       # [N, R]
    u = rng.standard_normal((w.batch, w.heads, rank, w.head_dim), dtype=np.float32)
    return np.float32(alpha) * np.einsum("nr,bhrd->bhnd", phi, u).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    """Q, K, V of one workload.  ``bits`` holds bf16 patterns (bf16 workloads)
    or float32 arrays (the fp32 workload); ``f32()`` returns exact float32."""

    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gk: Optional[np.ndarray] = None      # extra global rows [B, H, X, d] (text K)
    gv: Optional[np.ndarray] = None      # and their values

    @property
    def is_bf16(self) -> bool:
        return self.q.dtype == np.uint16

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bits_to_f32(a) if self.is_bf16 else a

    def torch(self, name: str, device="cuda"):
        import torch

        a = getattr(self, name)
        if self.is_bf16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)


def make_inputs(w: Workload, seed: Optional[int] = None, heads: Optional[int] = None) -> Inputs:
    """Draw a workload's Q, K, V (optionally with fewer heads for quick tests)."""
    if heads is not None:
        w = dataclasses.replace(w, heads=heads)
    seed = w.seed if seed is None else seed
    shape = (w.batch, w.heads, w.n_tokens, w.head_dim)
    q = _rng(seed, 0).standard_normal(shape, dtype=np.float32)
    k = _rng(seed, 1).standard_normal(shape, dtype=np.float32)
    v = _rng(seed, 2).standard_normal(shape, dtype=np.float32)
    if w.smooth:
        a = _smooth(w, _rng(seed, 3))
        q += a
        k += a
        del a
    gk = gv = None
    if w.text:
        gshape = (w.batch, w.heads, w.text, w.head_dim)
        gk = _rng(seed, 4).standard_normal(gshape, dtype=np.float32)
        gv = _rng(seed, 5).standard_normal(gshape, dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
        if w.text:
            gk, gv = bf16_bits(gk), bf16_bits(gv)
    return Inputs(w, q, k, v, gk, gv)


def make_grad(w: Workload, seed: Optional[int] = None, heads: Optional[int] = None) -> np.ndarray:
    """An incoming output gradient dO [B, H, N, d] for a backward pass, in the
    workload's storage (bf16 patterns or float32), standard normal."""
    if heads is not None:
        w = dataclasses.replace(w, heads=heads)
    seed = w.seed if seed is None else seed
    g = _rng(seed, 6).standard_normal((w.batch, w.heads, w.n_tokens, w.head_dim),
                                      dtype=np.float32)
    return bf16_bits(g) if w.dtype == "bf16" else g


def random_short_problem(rng: np.random.Generator, max_tokens: int = 600):
    """A random small problem whose window extents need not divide the grid
    (at least one does not); the pool divides the grid."""
    while True:
        grid = (int(rng.choice([1, 2, 3])), int(rng.choice([5, 6, 7, 9, 10])),
                int(rng.choice([6, 7, 10, 11, 13])))
        if np.prod(grid) > max_tokens:
            continue
        window = tuple(int(rng.integers(1, g + 1)) for g in grid)
        if all(g % w == 0 for g, w in zip(grid, window)):
            continue
        shift = tuple(int(rng.integers(0, g)) for g in grid)
        pool = tuple(int(rng.choice([d for d in range(1, g + 1) if g % d == 0])) for g in grid)
        return grid, window, shift, pool


def random_problem(rng: np.random.Generator, max_tokens: int = 768):
    """A random small divisible problem (grid, window, shift, pool) for property tests."""
    while True:
        T = int(rng.choice([1, 1, 2, 3, 4]))
        H = int(rng.choice([4, 6, 8, 12, 16]))
        W = int(rng.choice([4, 6, 8, 10, 12, 16]))
        if T * H * W > max_tokens:
            continue
        grid = (T, H, W)
        window = tuple(int(rng.choice([d for d in range(1, g + 1) if g % d == 0])) for g in grid)
        shift = tuple(int(rng.integers(0, g)) for g in grid)
        pool = tuple(int(rng.choice([d for d in range(1, g + 1) if g % d == 0])) for g in grid)
        return grid, window, shift, pool
