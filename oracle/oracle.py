"""ctypes binding of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It loads ``liboracle_basa.so`` built from
``basa_oracle.c`` (plain C, float64 arithmetic) and converts numpy arrays.

Method source: BASA (arXiv 2610.08772v1), paperlayer.ai summary, sections
3.1-3.3 and A.1-A.2; each C function cites the passage it follows.
``attend_text`` (the text queries of a joint block: dense attention over every
image token and text row) is written here in float64 numpy as its plain
definition; it is pinned by torch's float64 SDPA and by closed forms.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# BASA_ORACLE_LIBRARY names another build of the same source (the
# ASan/UBSan copy).
LIB_PATH = os.environ.get("BASA_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle_basa.so")
SOURCE = os.path.join(_HERE, "basa_oracle.c")

BO_OK, BO_EINVAL, BO_ENOTDIV, BO_ERANGE, BO_ENOMEM = range(5)


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


class _Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("grid", ctypes.c_int64 * 3),
        ("window", ctypes.c_int64 * 3),
        ("shift", ctypes.c_int64 * 3),
        ("pool", ctypes.c_int64 * 3),
        ("topk", ctypes.c_int64),
        ("scale", ctypes.c_double),
        ("radius", ctypes.c_int64),
        ("global_tokens", ctypes.c_int64),
    ]


@dataclasses.dataclass(frozen=True)
class Params:
    """One BASA block's attention problem as the oracle sees it."""

    batch: int
    heads: int
    dim: int
    grid: Sequence[int]
    window: Sequence[int]
    shift: Sequence[int] = (0, 0, 0)
    pool: Sequence[int] = (0, 0, 0)
    topk: int = 0
    scale: Optional[float] = None
    radius: int = -1
    global_tokens: int = 0

    def c(self) -> _Params:
        p = _Params()
        p.batch, p.heads, p.dim = self.batch, self.heads, self.dim
        for a in range(3):
            p.grid[a] = self.grid[a]
            p.window[a] = self.window[a]
            p.shift[a] = self.shift[a]
            p.pool[a] = self.pool[a]
        p.topk = self.topk
        p.radius = self.radius
        p.global_tokens = self.global_tokens
        if self.scale is not None:
            p.scale = self.scale
        else:
            p.scale = 1.0 / math.sqrt(self.dim) if self.dim > 0 else 1.0
        return p

    @property
    def n_tokens(self) -> int:
        return int(np.prod(self.grid))

    @property
    def n_windows(self) -> int:
        return int(np.prod([-(-g // w) for g, w in zip(self.grid, self.window)]))

    @property
    def padded(self) -> bool:
        return any(g % w for g, w in zip(self.grid, self.window))

    @property
    def window_tokens(self) -> int:
        return int(np.prod(self.window))

    @property
    def pooled_tokens(self) -> int:
        if not any(self.pool):
            return 0
        return int(np.prod([g // p for g, p in zip(self.grid, self.pool)]))

    @property
    def keys_per_query(self) -> int:
        return self.window_tokens * (1 + self.topk) + self.pooled_tokens + self.global_tokens

    @property
    def pool_on(self) -> bool:
        return any(self.pool)


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Params)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "bo_check": (ctypes.c_int, [P]),
        "bo_tokens": (ctypes.c_int64, [P]),
        "bo_windows": (ctypes.c_int64, [P]),
        "bo_window_tokens": (ctypes.c_int64, [P]),
        "bo_window_real_tokens": (ctypes.c_int64, [P, ctypes.c_int64]),
        "bo_pooled_tokens": (ctypes.c_int64, [P]),
        "bo_keys_per_query": (ctypes.c_int64, [P]),
        "bo_partition": (ctypes.c_int, [P, i32p, i32p, i32p]),
        "bo_pool": (ctypes.c_int, [P, f32p, f64p]),
        "bo_route": (ctypes.c_int, [P, f32p, f32p, i32p, f64p]),
        "bo_attend": (ctypes.c_int, [P, f32p, f32p, f32p, f64p, f64p, i32p, f64p, f64p]),
        "bo_attend_bwd": (ctypes.c_int, [P, f32p, f32p, f32p, f64p, f64p, i32p, f32p, f64p, f64p,
                                         f64p, f64p, f64p]),
        "bo_attend_bwd_dq_rows": (ctypes.c_int, [P, f32p, f32p, f32p, f64p, f64p, i32p, f32p,
                                                 ctypes.c_int64, i64p, f64p]),
        "bo_attend_bwd_window_keys": (ctypes.c_int, [P, f32p, f32p, f32p, f64p, f64p, i32p, f32p,
                                                     ctypes.c_int64, ctypes.c_int64, f64p, f64p]),
        "bo_attend_rows": (ctypes.c_int,
                           [P, f32p, f32p, f32p, f64p, f64p, i32p, ctypes.c_int64, i64p, f64p,
                            f64p]),
        "bo_softmax_row": (ctypes.c_int, [P, f32p, f32p, f64p, i32p, ctypes.c_int64, f64p, i64p]),
        "bo_num_threads": (ctypes.c_int, []),
        "bo_set_num_threads": (None, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _call(name: str, *args) -> None:
    rc = getattr(load(), name)(*args)
    if rc != BO_OK:
        raise OracleError(rc, name)


def check(p: Params) -> int:
    pc = p.c()
    return load().bo_check(ctypes.byref(pc))


def num_threads() -> int:
    return load().bo_num_threads()


def set_num_threads(n: int) -> None:
    load().bo_set_num_threads(int(n))


def window_real_tokens(p: Params) -> np.ndarray:
    """Slots of every window [nW] (M, or fewer for a short window)."""
    pc = p.c()
    f = load().bo_window_real_tokens
    return np.array([f(ctypes.byref(pc), w) for w in range(p.n_windows)], np.int64)


def partition(p: Params):
    """(win_id [N], slot [N], tok [nW, M]) of one block's window partition;
    tok is -1 past a short window's slots."""
    pc = p.c()
    n, nw, m = p.n_tokens, p.n_windows, p.window_tokens
    win_id = np.empty(n, np.int32)
    slot = np.empty(n, np.int32)
    tok = np.empty((nw, m), np.int32)
    _call("bo_partition", ctypes.byref(pc), _ptr(win_id, ctypes.c_int32),
          _ptr(slot, ctypes.c_int32), _ptr(tok, ctypes.c_int32))
    return win_id, slot, tok


def pool(p: Params, x: np.ndarray) -> np.ndarray:
    """Average-pooled memory [B, H, G, d] (float64) of x [B, H, N, d]."""
    pc = p.c()
    x = _f32(x)
    out = np.empty((p.batch, p.heads, p.pooled_tokens, p.dim), np.float64)
    _call("bo_pool", ctypes.byref(pc), _ptr(x, ctypes.c_float), _ptr(out, ctypes.c_double))
    return out


def route(p: Params, q: np.ndarray, k: np.ndarray, want_scores: bool = False):
    """Routed windows [B, H, nW, topk] (and optionally the score matrix)."""
    pc = p.c()
    q, k = _f32(q), _f32(k)
    r = np.empty((p.batch, p.heads, p.n_windows, max(p.topk, 0)), np.int32)
    sc = np.empty((p.batch, p.heads, p.n_windows, p.n_windows), np.float64) if want_scores else None
    _call("bo_route", ctypes.byref(pc), _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
          _ptr(r, ctypes.c_int32) if p.topk > 0 else None, _ptr(sc, ctypes.c_double))
    return (r, sc) if want_scores else r


def _prep_kv(p: Params, kp, vp, rt):
    kp = None if kp is None else np.ascontiguousarray(kp, np.float64)
    vp = None if vp is None else np.ascontiguousarray(vp, np.float64)
    rt = None if rt is None else np.ascontiguousarray(rt, np.int32)
    return kp, vp, rt


def attend(p: Params, q, k, v, kp=None, vp=None, rt=None):
    """Attention output [B, H, N, d] and lse [B, H, N], both float64."""
    pc = p.c()
    q, k, v = _f32(q), _f32(k), _f32(v)
    kp, vp, rt = _prep_kv(p, kp, vp, rt)
    out = np.empty((p.batch, p.heads, p.n_tokens, p.dim), np.float64)
    lse = np.empty((p.batch, p.heads, p.n_tokens), np.float64)
    _call("bo_attend", ctypes.byref(pc), _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
          _ptr(v, ctypes.c_float), _ptr(kp, ctypes.c_double), _ptr(vp, ctypes.c_double),
          _ptr(rt, ctypes.c_int32), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return out, lse


def attend_rows(p: Params, q, k, v, rows: np.ndarray, kp=None, vp=None, rt=None):
    """Attention output for selected rows ((b*H + h)*N + n): out [R, d], lse [R]."""
    pc = p.c()
    q, k, v = _f32(q), _f32(k), _f32(v)
    kp, vp, rt = _prep_kv(p, kp, vp, rt)
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, p.dim), np.float64)
    lse = np.empty(rows.size, np.float64)
    _call("bo_attend_rows", ctypes.byref(pc), _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
          _ptr(v, ctypes.c_float), _ptr(kp, ctypes.c_double), _ptr(vp, ctypes.c_double),
          _ptr(rt, ctypes.c_int32), ctypes.c_int64(rows.size), _ptr(rows, ctypes.c_int64),
          _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return out, lse


def softmax_row(p: Params, q, k, row: int, kp=None, rt=None):
    """Softmax probabilities of one query over its key list, and each key's source."""
    pc = p.c()
    q, k = _f32(q), _f32(k)
    kp, _, rt = _prep_kv(p, kp, None, rt)
    probs = np.empty(p.keys_per_query, np.float64)
    key_id = np.empty(p.keys_per_query, np.int64)
    _call("bo_softmax_row", ctypes.byref(pc), _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
          _ptr(kp, ctypes.c_double), _ptr(rt, ctypes.c_int32), ctypes.c_int64(row),
          _ptr(probs, ctypes.c_double), _ptr(key_id, ctypes.c_int64))
    return probs, key_id


def attend_bwd(p: Params, q, k, v, dout, kp=None, vp=None, rt=None):
    """Gradients of the block's output for the incoming gradient dout:
    dict(dq, dk, dv [B, H, N, d], dkg, dvg [B, H, G + X, d] or None), float64.
    dk, dv include the pooled cells' share carried back to their tokens."""
    pc = p.c()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    kp, vp, rt = _prep_kv(p, kp, vp, rt)
    shape = (p.batch, p.heads, p.n_tokens, p.dim)
    dq, dk, dv = np.empty(shape), np.empty(shape), np.empty(shape)
    g = p.pooled_tokens + p.global_tokens
    dkg = np.empty((p.batch, p.heads, g, p.dim)) if g else None
    dvg = np.empty((p.batch, p.heads, g, p.dim)) if g else None
    _call("bo_attend_bwd", ctypes.byref(pc), _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
          _ptr(v, ctypes.c_float), _ptr(kp, ctypes.c_double), _ptr(vp, ctypes.c_double),
          _ptr(rt, ctypes.c_int32), _ptr(dout, ctypes.c_float), _ptr(dq, ctypes.c_double),
          _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double), _ptr(dkg, ctypes.c_double),
          _ptr(dvg, ctypes.c_double))
    return dict(dq=dq, dk=dk, dv=dv, dkg=dkg, dvg=dvg)


def attend_bwd_dq_rows(p: Params, q, k, v, dout, rows: np.ndarray, kp=None, vp=None, rt=None):
    """dq of selected query rows ((b*H + h)*N + n): [R, d] float64."""
    pc = p.c()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    kp, vp, rt = _prep_kv(p, kp, vp, rt)
    rows = np.ascontiguousarray(rows, np.int64)
    dq = np.empty((rows.size, p.dim), np.float64)
    _call("bo_attend_bwd_dq_rows", ctypes.byref(pc), _ptr(q, ctypes.c_float),
          _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), _ptr(kp, ctypes.c_double),
          _ptr(vp, ctypes.c_double), _ptr(rt, ctypes.c_int32), _ptr(dout, ctypes.c_float),
          ctypes.c_int64(rows.size), _ptr(rows, ctypes.c_int64), _ptr(dq, ctypes.c_double))
    return dq


def attend_bwd_window_keys(p: Params, q, k, v, dout, bh: int, w: int, kp=None, vp=None, rt=None):
    """Key gradients (dk, dv [M, d], float64, slot order) of window w's tokens
    at bh = b*H + h, before the pooled cells' share is carried back."""
    pc = p.c()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    kp, vp, rt = _prep_kv(p, kp, vp, rt)
    dk = np.empty((p.window_tokens, p.dim), np.float64)
    dv = np.empty((p.window_tokens, p.dim), np.float64)
    _call("bo_attend_bwd_window_keys", ctypes.byref(pc), _ptr(q, ctypes.c_float),
          _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), _ptr(kp, ctypes.c_double),
          _ptr(vp, ctypes.c_double), _ptr(rt, ctypes.c_int32), _ptr(dout, ctypes.c_float),
          ctypes.c_int64(bh), ctypes.c_int64(w), _ptr(dk, ctypes.c_double),
          _ptr(dv, ctypes.c_double))
    return dk, dv


def global_rows(p: Params, x, extra=None):
    """The global part of the key list [B, H, G + X, d] (float64): the pooled
    cells of x, then the X extra rows `extra` ([B, H, X, d]); None if empty."""
    parts = []
    if p.pool_on:
        parts.append(pool(p, x))
    if p.global_tokens:
        parts.append(np.asarray(extra, np.float64))
    return np.concatenate(parts, axis=2) if parts else None


def forward(p: Params, q, k, v, gk=None, gv=None):
    """The whole block as the method defines it: pool, route, attend.  gk, gv:
    the extra global rows (e.g. text K/V) when p.global_tokens > 0."""
    kp = global_rows(p, k, gk)
    vp = global_rows(p, v, gv)
    rt = route(p, q, k) if p.topk > 0 else None
    out, lse = attend(p, q, k, v, kp, vp, rt)
    return dict(out=out, lse=lse, kp=kp, vp=vp, route=rt)


def attend_text(p: Params, q_text, k, v, k_text, v_text):
    """Text queries of a joint block (the pages' A.1 takes the text tokens as a
    branch of the image queries' softmax and says nothing of the text tokens'
    own queries; read plainly they attend densely): for every (b, h) and text
    row s, out[s] = softmax(scale * q_text[s] . [K ++ K_text]^T) [V ++ V_text]
    over all N image tokens and the X text rows, in float64, shifted by the
    row maximum.  Returns out [B, H, X, d] and the natural-log lse [B, H, X]."""
    scale = p.scale if p.scale is not None else 1.0 / math.sqrt(p.dim)
    q = np.asarray(q_text, np.float64)
    keys = np.concatenate([np.asarray(k, np.float64), np.asarray(k_text, np.float64)], axis=2)
    vals = np.concatenate([np.asarray(v, np.float64), np.asarray(v_text, np.float64)], axis=2)
    logits = scale * (q @ np.swapaxes(keys, 2, 3))
    m = logits.max(axis=3, keepdims=True)
    e = np.exp(logits - m)
    total = e.sum(axis=3, keepdims=True)
    out = (e @ vals) / total
    return out, (m + np.log(total))[..., 0]



def shift_schedule(window, layer: int, step: int, n_offsets: int, axes=(1, 2)):
    """Shift of block `layer` at denoising step `step` (paperlayer.ai summary,
    sec. 3.1: candidate offsets interleave across layers, then advance across
    denoising steps).  Reading: n_offsets evenly spaced candidates per offset
    axis, candidate c = c * window // n_offsets; layer l at step s uses
    candidate (l + s) mod n_offsets; axes not in `axes` keep offset 0."""
    candidates = [[c * int(window[a]) // n_offsets for c in range(n_offsets)] for a in range(3)]
    c = (layer + step) % n_offsets
    return tuple(candidates[a][c] if a in axes else 0 for a in range(3))


def key_list_pairs(p: Params, rt=None) -> int:
    """Total (query, key) pairs of a forward: for every head and window, each
    of its real tokens attends to the window's real tokens, the G + X global
    rows and the real tokens of each routed window (A.1's concatenated key
    list), summed over the key lists' lengths."""
    mw = window_real_tokens(p)
    g = p.pooled_tokens + p.global_tokens
    total = 0
    for bh in range(p.batch * p.heads):
        for w in range(p.n_windows):
            keys = int(mw[w]) + g
            if p.topk > 0:
                b, h = divmod(bh, p.heads)
                keys += sum(int(mw[j]) for j in rt[b, h, w])
            total += int(mw[w]) * keys
    return total
