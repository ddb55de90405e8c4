"""Efficiency metrics as the BASA pages define them (thelatestinai.com card,
Table 3; the paperlayer.ai summary, sec. 4.2 and A.1).

* FLOPs of an attention call: (query, key) pairs times the work per pair.  The
  pages' Table 3 counts 4d + 3 per pair (two d-long products plus three
  scalar softmax operations); this library reports 4d (the matrix-core work).
* MFU: FLOPs / latency / peak.
* Kernel efficiency (the tables' "Kernel Eff." and "Real."): measured speedup
  over dense divided by the theoretical FLOP ratio, i.e. MFU_sparse / MFU_dense.
"""
from __future__ import annotations

# Dense bf16 matrix-core peak of one MI355X (AMD's published figure).
MI355X_BF16_PEAK = 2.5e15
# HBM3E bandwidth of one MI355X (published).
MI355X_HBM_PEAK = 8.0e12
# The 16-bit tensor peak the pages' MFU column implies (one A100).
A100_16BIT_PEAK = 312e12


def attention_flops(pairs: float, head_dim: int, extra_per_pair: int = 0) -> float:
    return pairs * (4 * head_dim + extra_per_pair)


def mfu(flops: float, seconds: float, peak: float) -> float:
    return flops / seconds / peak


def speedup(t_dense: float, t_sparse: float) -> float:
    return t_dense / t_sparse


def kernel_efficiency(t_dense: float, t_sparse: float, f_dense: float, f_sparse: float) -> float:
    return speedup(t_dense, t_sparse) / (f_dense / f_sparse)
