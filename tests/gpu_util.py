"""Helpers shared by the GPU parity tests: plans from workloads, comparisons."""
from __future__ import annotations

import sys

import numpy as np

from oracle.oracle import Params
from video_gen_amd.synth import Workload

# Tolerances for bf16 attention output against the float64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 2e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_params(w: Workload, shift, heads=None, dense=False) -> Params:
    h = w.heads if heads is None else heads
    if dense:
        return Params(w.batch, h, w.head_dim, w.grid, w.grid, (0, 0, 0), (0, 0, 0), 0)
    return Params(w.batch, h, w.head_dim, w.grid, w.window, shift, w.pool, w.topk,
                  radius=w.radius, global_tokens=w.text)


def basa_plan(basa, w: Workload, shift, heads=None, dense=False):
    h = w.heads if heads is None else heads
    if dense:
        return basa.Plan(w.batch, h, w.head_dim, w.grid, w.grid, (0, 0, 0), (0, 0, 0), 0, w.dtype)
    return basa.Plan(w.batch, h, w.head_dim, w.grid, w.window, shift, w.pool, w.topk, w.dtype,
                     route_radius=w.radius, global_tokens=w.text)


def to_f64(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def compare(got: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"  {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err.max() <= max_abs, f"{what}: max abs error {err.max():.3e} > {max_abs}"
    assert err.mean() <= mean_abs, f"{what}: mean abs error {err.mean():.3e} > {mean_abs}"
    return err, rel


# Query slots per attention workgroup (the largest the kernel takes): the
# sampled rows cover a window's whole last tile of this size.
QUERY_TILE = 256


def sample_rows(w: Workload, tok: np.ndarray, heads: int, n_random: int, seed: int) -> np.ndarray:
    """Flat row ids (b*H + h)*N + n: random rows plus every slot of one window's
    last (ragged) query tile and the first/last slot of a few windows."""
    rng = np.random.default_rng(seed)
    N = w.n_tokens
    total = w.batch * heads * N
    rows = set(rng.integers(0, total, size=n_random).tolist())
    nw = tok.shape[0]
    mw = (tok >= 0).sum(axis=1)            # short windows end in -1 entries
    for bh in (0, w.batch * heads - 1):
        for wi in (int(rng.integers(0, nw)), nw - 1):
            m = int(mw[wi])
            last_tile = (m - 1) // QUERY_TILE * QUERY_TILE
            for s in range(last_tile, m):
                rows.add(bh * N + int(tok[wi, s]))
        for wj in (0, nw - 1, int(rng.integers(0, nw))):
            rows.add(bh * N + int(tok[wj, 0]))
            rows.add(bh * N + int(tok[wj, int(mw[wj]) - 1]))
    return np.array(sorted(rows), np.int64)
