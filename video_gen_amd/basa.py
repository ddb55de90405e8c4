"""ctypes binding of libbasa (argument marshalling only).

The functions carry the C names declared in ``include/basa.h``; each takes
torch tensors that already live on the GPU, checks their dtype, shape and
contiguity, and passes raw device pointers plus torch's current HIP stream to
the library.  Every step of the computation runs in libbasa's HIP kernels;
there is no fallback: if the library is missing, loading it raises.

Import torch before this module is used: torch's HIP runtime then serves the
library as well (one runtime per process).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
# BASA_LIBRARY names another build of the same library (the host-sanitized
# copy that ``build.build(sanitize=True)`` writes).
LIB_PATH = os.environ.get("BASA_LIBRARY") or os.path.join(PKG, "libbasa.so")

BASA_OK = 0
BASA_ERR_INVALID_ARGUMENT = 1
BASA_ERR_NOT_DIVISIBLE = 2
BASA_ERR_UNSUPPORTED = 3
BASA_ERR_HIP = 4
BASA_ERR_OUT_OF_MEMORY = 5
BASA_BF16 = 0
BASA_F32 = 1

EXPORTED = ("basa_plan", "basa_plan_destroy", "basa_plan_get_info", "basa_plan_pairs",
            "basa_shift_schedule", "basa_pool_kv",
            "basa_route_windows", "basa_route_windows_noalloc", "basa_window_attn_fwd",
            "basa_text_attn_fwd",
            "basa_window_attn_fwd_split",
            "basa_window_attn_bwd",
            "basa_window_index",
            "basa_gather_windows", "basa_probe_mfma", "basa_status_string", "basa_last_error")


class BasaError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: {status_string(status)}: {detail}")
        self.status = status


class _Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("grid", ctypes.c_int32 * 3), ("window", ctypes.c_int32 * 3),
        ("shift", ctypes.c_int32 * 3), ("pool", ctypes.c_int32 * 3),
        ("route_topk", ctypes.c_int32), ("route_radius", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("softmax_scale", ctypes.c_float),
        ("global_tokens", ctypes.c_int32),
    ]


class _Info(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64), ("n_windows", ctypes.c_int64),
        ("window_tokens", ctypes.c_int64), ("pooled_tokens", ctypes.c_int64),
        ("keys_per_query", ctypes.c_int64), ("route_workspace_bytes", ctypes.c_int64),
        ("pairs_sparse", ctypes.c_double), ("pairs_dense", ctypes.c_double),
        ("flops_sparse", ctypes.c_double), ("flops_dense", ctypes.c_double),
        ("global_tokens", ctypes.c_int64), ("bwd_workspace_bytes", ctypes.c_int64),
        ("split_workspace_bytes", ctypes.c_int64), ("text_splits", ctypes.c_int64),
        ("text_workspace_bytes", ctypes.c_int64),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbasa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} not found: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    st = ctypes.c_int
    sig = {
        "basa_plan": (st, [ctypes.POINTER(_Params), ctypes.POINTER(vp)]),
        "basa_plan_destroy": (None, [vp]),
        "basa_plan_get_info": (st, [vp, ctypes.POINTER(_Info)]),
        "basa_plan_pairs": (st, [vp, vp, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]),
        "basa_shift_schedule": (st, [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32)]),
        "basa_pool_kv": (st, [vp, vp, vp, vp, vp, vp]),
        "basa_route_windows": (st, [vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "basa_route_windows_noalloc": (st, [vp, vp, vp, vp, vp]),
        "basa_window_attn_fwd": (st, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "basa_text_attn_fwd": (st, [vp] * 9 + [ctypes.c_size_t, vp]),
        "basa_window_attn_fwd_split": (st, [vp] * 9 + [ctypes.c_int, vp, ctypes.c_size_t, vp]),
        "basa_window_attn_bwd": (st, [vp] * 16 + [ctypes.c_size_t, vp]),
        "basa_window_index": (st, [vp, vp, vp, vp]),
        "basa_gather_windows": (st, [vp, vp, vp, vp]),
        "basa_probe_mfma": (st, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                 ctypes.POINTER(ctypes.c_double), vp]),
        "basa_status_string": (ctypes.c_char_p, [st]),
        "basa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().basa_status_string(status).decode()


def last_error() -> str:
    return load().basa_last_error().decode()


def _check(status: int, fn: str) -> None:
    if status != BASA_OK:
        raise BasaError(status, fn, last_error())


class Plan:
    """An immutable libbasa plan for one block (one shift)."""

    def __init__(self, batch: int, heads: int, head_dim: int, grid: Sequence[int],
                 window: Sequence[int], shift: Sequence[int] = (0, 0, 0),
                 pool: Sequence[int] = (0, 0, 0), route_topk: int = 0, dtype: str = "bf16",
                 softmax_scale: float = 0.0, route_radius: int = -1, global_tokens: int = 0):
        lib = load()
        p = _Params()
        p.batch, p.heads, p.head_dim = batch, heads, head_dim
        for a in range(3):
            p.grid[a], p.window[a] = grid[a], window[a]
            p.shift[a], p.pool[a] = shift[a], pool[a]
        p.route_topk, p.route_radius = route_topk, route_radius
        p.dtype = {"bf16": BASA_BF16, "f32": BASA_F32}[dtype]
        p.softmax_scale = softmax_scale
        p.global_tokens = global_tokens
        h = ctypes.c_void_p()
        _check(lib.basa_plan(ctypes.byref(p), ctypes.byref(h)), "basa_plan")
        self._h = h
        self.params = dict(batch=batch, heads=heads, head_dim=head_dim, grid=tuple(grid),
                           window=tuple(window), shift=tuple(shift), pool=tuple(pool),
                           route_topk=route_topk, dtype=dtype, route_radius=route_radius,
                           global_tokens=global_tokens)
        info = _Info()
        _check(lib.basa_plan_get_info(h, ctypes.byref(info)), "basa_plan_get_info")
        self.info = {f: getattr(info, f) for f, _ in _Info._fields_}

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.basa_plan_destroy(h)
            self._h = None

    # shapes the entry points expect
    @property
    def token_shape(self):
        p = self.params
        return (p["batch"], p["heads"], self.info["n_tokens"], p["head_dim"])

    @property
    def pooled_shape(self):
        """Shape of k_pool / v_pool: the G pooled cells, then the X extra
        global rows."""
        p = self.params
        return (p["batch"], p["heads"], self.info["pooled_tokens"] + self.info["global_tokens"],
                p["head_dim"])

    @property
    def text_shape(self):
        """Shape of the text queries and their output: the X extra global rows."""
        p = self.params
        return (p["batch"], p["heads"], self.info["global_tokens"], p["head_dim"])

    @property
    def route_shape(self):
        p = self.params
        return (p["batch"], p["heads"], self.info["n_windows"], p["route_topk"])


def shift_schedule(window: Sequence[int], layer: int, step: int, n_offsets: int = 2,
                   axes: Sequence[int] = (1, 2)) -> Tuple[int, int, int]:
    """Cyclic partition offset of block `layer` at denoising step `step`
    (basa_shift_schedule: candidate offsets interleaved over the layers and
    advanced by one per step along `axes`)."""
    w = (ctypes.c_int32 * 3)(*[int(x) for x in window])
    out = (ctypes.c_int32 * 3)()
    mask = sum(1 << int(a) for a in axes)
    _check(load().basa_shift_schedule(w, int(layer), int(step), int(n_offsets), mask, out),
           "basa_shift_schedule")
    return tuple(int(x) for x in out)


def plan_pairs(plan: "Plan", route_host=None) -> Tuple[float, float]:
    """(pairs, flops) a forward of `plan` computes with the given route table
    (a host int32 array [B, H, nW, topk], or None when the plan does not
    route): basa_plan_pairs."""
    import numpy as np

    rt = None
    if route_host is not None:
        route_host = np.ascontiguousarray(route_host, dtype=np.int32)
        if route_host.shape != tuple(plan.route_shape):
            raise ValueError(f"route has shape {route_host.shape}, expected {plan.route_shape}")
        rt = route_host.ctypes.data_as(ctypes.c_void_p)
    pairs, flops = ctypes.c_double(), ctypes.c_double()
    _check(load().basa_plan_pairs(plan.handle, rt, ctypes.byref(pairs), ctypes.byref(flops)),
           "basa_plan_pairs")
    return pairs.value, flops.value


def basa_plan(**kw) -> Plan:
    return Plan(**kw)


def _torch():
    import torch

    return torch


def _dev(t, shape, dtype, name):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _elem(plan: Plan):
    torch = _torch()
    return torch.bfloat16 if plan.params["dtype"] == "bf16" else torch.float32


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def basa_pool_kv(plan: Plan, k, v, k_pool, v_pool, stream=None) -> None:
    e = _elem(plan)
    _check(load().basa_pool_kv(plan.handle, _dev(k, plan.token_shape, e, "k"),
                               _dev(v, plan.token_shape, e, "v"),
                               _dev(k_pool, plan.pooled_shape, e, "k_pool"),
                               _dev(v_pool, plan.pooled_shape, e, "v_pool"), _stream(stream)),
           "basa_pool_kv")


def basa_route_windows(plan: Plan, q, k, route, workspace, stream=None) -> None:
    torch = _torch()
    e = _elem(plan)
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().basa_route_windows(plan.handle, _dev(q, plan.token_shape, e, "q"),
                                     _dev(k, plan.token_shape, e, "k"),
                                     _dev(route, plan.route_shape, torch.int32, "route"),
                                     ctypes.c_void_p(workspace.data_ptr()), nbytes,
                                     _stream(stream)),
           "basa_route_windows")


def basa_route_windows_noalloc(plan: Plan, q, k, route, stream=None) -> None:
    """Routing with the library's own per-GPU scratch (no workspace)."""
    torch = _torch()
    e = _elem(plan)
    _check(load().basa_route_windows_noalloc(plan.handle, _dev(q, plan.token_shape, e, "q"),
                                             _dev(k, plan.token_shape, e, "k"),
                                             _dev(route, plan.route_shape, torch.int32, "route"),
                                             _stream(stream)),
           "basa_route_windows_noalloc")


def basa_window_attn_fwd(plan: Plan, q, k, v, k_pool, v_pool, route, out, lse=None,
                         stream=None) -> None:
    torch = _torch()
    e = _elem(plan)
    kp = _dev(k_pool, plan.pooled_shape, e, "k_pool") if k_pool is not None else None
    vpp = _dev(v_pool, plan.pooled_shape, e, "v_pool") if v_pool is not None else None
    rt = _dev(route, plan.route_shape, torch.int32, "route") if route is not None else None
    ls = (_dev(lse, plan.token_shape[:3], torch.float32, "lse") if lse is not None else None)
    _check(load().basa_window_attn_fwd(plan.handle, _dev(q, plan.token_shape, e, "q"),
                                       _dev(k, plan.token_shape, e, "k"),
                                       _dev(v, plan.token_shape, e, "v"), kp, vpp, rt,
                                       _dev(out, plan.token_shape, e, "out"), ls,
                                       _stream(stream)),
           "basa_window_attn_fwd")


def basa_text_attn_fwd(plan: Plan, q_text, k, v, k_global, v_global, out_text, lse_text=None,
                       workspace=None, stream=None) -> None:
    """Text queries of a joint block: dense over every image token and text
    row.  workspace: a contiguous GPU tensor of at least
    info["text_workspace_bytes"] bytes when that is nonzero."""
    torch = _torch()
    e = _elem(plan)
    ls = (_dev(lse_text, plan.text_shape[:3], torch.float32, "lse_text")
          if lse_text is not None else None)
    ws, nbytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        ws, nbytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    _check(load().basa_text_attn_fwd(plan.handle, _dev(q_text, plan.text_shape, e, "q_text"),
                                     _dev(k, plan.token_shape, e, "k"),
                                     _dev(v, plan.token_shape, e, "v"),
                                     _dev(k_global, plan.pooled_shape, e, "k_global"),
                                     _dev(v_global, plan.pooled_shape, e, "v_global"),
                                     _dev(out_text, plan.text_shape, e, "out_text"), ls, ws,
                                     nbytes, _stream(stream)),
           "basa_text_attn_fwd")


def basa_window_attn_fwd_split(plan: Plan, q, k, v, k_pool, v_pool, route, out, lse, ways,
                               workspace, stream=None) -> None:
    torch = _torch()
    e = _elem(plan)
    kp = _dev(k_pool, plan.pooled_shape, e, "k_pool") if k_pool is not None else None
    vpp = _dev(v_pool, plan.pooled_shape, e, "v_pool") if v_pool is not None else None
    rt = _dev(route, plan.route_shape, torch.int32, "route") if route is not None else None
    ls = (_dev(lse, plan.token_shape[:3], torch.float32, "lse") if lse is not None else None)
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().basa_window_attn_fwd_split(
        plan.handle, _dev(q, plan.token_shape, e, "q"), _dev(k, plan.token_shape, e, "k"),
        _dev(v, plan.token_shape, e, "v"), kp, vpp, rt, _dev(out, plan.token_shape, e, "out"), ls,
        int(ways), ctypes.c_void_p(workspace.data_ptr()), nbytes, _stream(stream)),
        "basa_window_attn_fwd_split")


def basa_window_attn_bwd(plan: Plan, q, k, v, k_pool, v_pool, route, out, lse, d_out,
                         d_q, d_k, d_v, d_k_global, d_v_global, workspace,
                         stream=None) -> None:
    torch = _torch()
    e, f = _elem(plan), torch.float32
    ts = plan.token_shape
    opt = lambda t, shape, dt, name: _dev(t, shape, dt, name) if t is not None else None
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().basa_window_attn_bwd(
        plan.handle, _dev(q, ts, e, "q"), _dev(k, ts, e, "k"), _dev(v, ts, e, "v"),
        opt(k_pool, plan.pooled_shape, e, "k_pool"), opt(v_pool, plan.pooled_shape, e, "v_pool"),
        opt(route, plan.route_shape, torch.int32, "route"), _dev(out, ts, e, "out"),
        _dev(lse, ts[:3], f, "lse"), _dev(d_out, ts, e, "d_out"), _dev(d_q, ts, f, "d_q"),
        _dev(d_k, ts, f, "d_k"), _dev(d_v, ts, f, "d_v"),
        opt(d_k_global, plan.pooled_shape, f, "d_k_global"),
        opt(d_v_global, plan.pooled_shape, f, "d_v_global"),
        ctypes.c_void_p(workspace.data_ptr()), nbytes, _stream(stream)),
        "basa_window_attn_bwd")


def basa_window_index(plan: Plan, win_id, slot, stream=None) -> None:
    torch = _torch()
    n = (plan.info["n_tokens"],)
    _check(load().basa_window_index(plan.handle, _dev(win_id, n, torch.int32, "win_id"),
                                    _dev(slot, n, torch.int32, "slot"), _stream(stream)),
           "basa_window_index")


def basa_gather_windows(plan: Plan, x, x_win, stream=None) -> None:
    e = _elem(plan)
    p = plan.params
    wshape = (p["batch"], p["heads"], plan.info["n_windows"], plan.info["window_tokens"],
              p["head_dim"])
    _check(load().basa_gather_windows(plan.handle, _dev(x, plan.token_shape, e, "x"),
                                      _dev(x_win, wshape, e, "x_win"), _stream(stream)),
           "basa_gather_windows")


def basa_probe_mfma(iters: int, n_workgroups: int, sink, clocks, mode: int = 0,
                    stream=None) -> float:
    """Matrix-core probe launch (measurement hook); returns its flop count.
    sink: float32 [n_workgroups * 256], clocks: int64 [n_workgroups, 4];
    mode 0 constant operands, 1 switching operands."""
    torch = _torch()
    n = int(n_workgroups)
    flops = ctypes.c_double(0.0)
    _check(load().basa_probe_mfma(int(iters), int(mode), n,
                                  _dev(sink, (n * 256,), torch.float32, "sink"),
                                  _dev(clocks, (n, 4), torch.int64, "clocks"),
                                  ctypes.byref(flops), _stream(stream)),
           "basa_probe_mfma")
    return flops.value


# ----------------------------------------------------------- convenience

# Execution chosen per static shape by Block(execution="auto"), as the pages'
# warm-up does (paperlayer.ai, A.1): plan parameters -> "fused" | "split2" | "split3".
_EXECUTION_CACHE: dict = {}
EXECUTIONS = ("fused", "split2", "split3")


class Block:
    """Device buffers and plans for one BASA block: pool -> route -> attend.

    Allocates the pooled K/V, the route table, its workspace and the output
    once (torch caching allocator); ``forward`` then enqueues only libbasa
    kernels on the current stream.  ``execution`` picks the attention's
    form: "fused" (one pass over the joint key list), "split2" / "split3"
    (branches merged by log-sum-exp), or "auto": on the first forward each
    form is timed on the block's own inputs and the fastest is cached for
    the plan's shape.
    """

    def __init__(self, plan: Plan, device="cuda", execution: str = "fused"):
        torch = _torch()
        if execution not in EXECUTIONS + ("auto",):
            raise ValueError(f"execution must be one of {EXECUTIONS + ('auto',)}")
        self.execution = execution
        self.split_ws = None
        self.plan = plan
        e = _elem(plan)
        info = plan.info
        self.k_pool = self.v_pool = None
        if info["pooled_tokens"] + info["global_tokens"] > 0:
            self.k_pool = torch.empty(plan.pooled_shape, dtype=e, device=device)
            self.v_pool = torch.empty(plan.pooled_shape, dtype=e, device=device)
        self.route = self.workspace = None
        if plan.params["route_topk"] > 0:
            self.route = torch.empty(plan.route_shape, dtype=torch.int32, device=device)
            nbytes = info["route_workspace_bytes"]
            self.workspace = torch.empty(max(1, math.ceil(nbytes / 8)), dtype=torch.float64,
                                         device=device)
        self.out = torch.empty(plan.token_shape, dtype=e, device=device)

    def set_global(self, k_rows, v_rows) -> None:
        """Places the X extra global K/V rows ([B, H, X, d], e.g. text tokens)
        after the pooled cells; they stay until set again."""
        g = self.plan.info["pooled_tokens"]
        self.k_pool[:, :, g:].copy_(k_rows)
        self.v_pool[:, :, g:].copy_(v_rows)

    def text_forward(self, q_text, k, v, lse_text=None):
        """Text queries of the joint block ([B, H, X, d]) over every image token
        and the text rows placed by set_global; returns out_text."""
        torch = _torch()
        if getattr(self, "out_text", None) is None:
            self.out_text = torch.empty(self.plan.text_shape, dtype=_elem(self.plan),
                                        device=self.out.device)
            nbytes = self.plan.info["text_workspace_bytes"]
            self.text_ws = (torch.empty(math.ceil(nbytes / 8), dtype=torch.float64,
                                        device=self.out.device) if nbytes else None)
        basa_text_attn_fwd(self.plan, q_text, k, v, self.k_pool, self.v_pool, self.out_text,
                           lse_text, self.text_ws)
        return self.out_text

    def _attend(self, how, q, k, v, lse):
        if how == "fused":
            basa_window_attn_fwd(self.plan, q, k, v, self.k_pool, self.v_pool, self.route,
                                 self.out, lse)
            return
        if self.split_ws is None:
            nbytes = self.plan.info["split_workspace_bytes"]
            self.split_ws = _torch().empty(max(1, math.ceil(nbytes / 8)), dtype=_torch().float64,
                                           device=self.out.device)
        basa_window_attn_fwd_split(self.plan, q, k, v, self.k_pool, self.v_pool, self.route,
                                   self.out, lse, 2 if how == "split2" else 3, self.split_ws)

    def _select(self, q, k, v, lse, reps=3):
        """Times each form on these inputs (HIP events) and caches the fastest."""
        torch = _torch()
        key = tuple(sorted(self.plan.params.items()))
        if key not in _EXECUTION_CACHE:
            best = None
            for how in EXECUTIONS:
                self._attend(how, q, k, v, lse)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    self._attend(how, q, k, v, lse)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                if best is None or ms < best[0]:
                    best = (ms, how)
            _EXECUTION_CACHE[key] = best[1]
        return _EXECUTION_CACHE[key]

    def forward(self, q, k, v, lse=None):
        if self.plan.info["pooled_tokens"] > 0:
            basa_pool_kv(self.plan, k, v, self.k_pool, self.v_pool)
        if self.route is not None:
            basa_route_windows(self.plan, q, k, self.route, self.workspace)
        how = self.execution
        if how == "auto":
            how = self._select(q, k, v, lse)
        self._attend(how, q, k, v, lse)
        return self.out

    def backward(self, q, k, v, lse, d_out):
        """Gradients after ``forward(q, k, v, lse)`` (same inputs, its lse):
        returns float32 (d_q, d_k, d_v, d_k_global, d_v_global); the last two
        are None without global rows.  Buffers are allocated on the first
        call and reused."""
        torch = _torch()
        if getattr(self, "d_q", None) is None:
            dev, f = self.out.device, torch.float32
            self.d_q = torch.empty(self.plan.token_shape, dtype=f, device=dev)
            self.d_k = torch.empty_like(self.d_q)
            self.d_v = torch.empty_like(self.d_q)
            self.d_kg = self.d_vg = None
            if self.k_pool is not None:
                self.d_kg = torch.empty(self.plan.pooled_shape, dtype=f, device=dev)
                self.d_vg = torch.empty_like(self.d_kg)
            nbytes = self.plan.info["bwd_workspace_bytes"]
            self.bwd_ws = torch.empty(max(1, math.ceil(nbytes / 8)), dtype=torch.float64,
                                      device=dev)
        basa_window_attn_bwd(self.plan, q, k, v, self.k_pool, self.v_pool, self.route, self.out,
                             lse, d_out, self.d_q, self.d_k, self.d_v, self.d_kg, self.d_vg,
                             self.bwd_ws)
        return self.d_q, self.d_k, self.d_v, self.d_kg, self.d_vg
