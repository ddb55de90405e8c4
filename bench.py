#!/usr/bin/env python3
"""Benchmark of the BASA attention forward (libbasa on one MI355X).

A step is one pass of the hot path over one batch of synthetic input: two
consecutive DiT blocks of the workload -- the even block (shift 0) and the
odd block (shift s) -- each running pool -> [route] -> window attention.
The same kernel is also timed dense (window = whole grid, no pooling, no
routing) to give the measured speedup and its ratio to the theoretical FLOP
ratio (the pages' "Kernel Eff." / "Real."; thelatestinai.com card, Tables 2
and 3), and the attention backward of the odd block is timed on its own
(the "backward" object; the pages adapt the model by training through it).
Video workloads (default "wan", and "wan_t3": Wan2.1 1664x960 at the
pages' Table 3 shape) are timed the same way beside the main one, the first
under "video", the others under "video_more".  FLOP counts take routed windows at their real
sizes (from the route table the timed run wrote).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("BASA attn fwd ms + TFLOP/s (% bf16 MFMA peak); "
          "measured/theoretical speedup vs dense")
DEFAULT_WORKLOAD = "flux2k"
ATTN_KERNEL = "window_attn_fwd_kernel"
ATTN_SOURCES = ("k_attn.hip", "device_common.hpp", "basa_internal.hpp")


def _r(x, nd):
    return None if x is None else round(x, nd)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--dense-reps", type=int, default=10)
    ap.add_argument("--bwd-reps", type=int, default=10,
                    help="timed calls of the attention backward (0 skips it)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--video-workload", default="wan,wan_t3",
                    help="comma-separated video workloads timed beside the main one "
                         "('none' skips them); the first is reported under 'video', "
                         "the rest under 'video_more'")
    ap.add_argument("--flush-reps", type=int, default=10,
                    help="attention launches timed with the caches emptied first (0 skips)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the matrix-core probe (e.g. under a counter run)")
    return ap.parse_args()


def attn_source_sha() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "video_gen_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != attn_source_sha():
        return None
    return float(val.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def tiny_one_thread(O):
    """The whole tiny block (pool, then attention of every query; odd shift)
    on one thread, for a per-core figure."""
    from video_gen_amd.synth import WORKLOADS, make_inputs

    w = WORKLOADS["tiny"]
    inp = make_inputs(w)
    p = O.Params(w.batch, w.heads, w.head_dim, w.grid, w.window, w.shift, w.pool, w.topk)
    O.set_num_threads(1)
    t0 = time.perf_counter()
    O.forward(p, inp.f32("q"), inp.f32("k"), inp.f32("v"))
    dt = time.perf_counter() - t0
    flops = 4.0 * w.head_dim * p.keys_per_query * w.n_tokens * w.batch * w.heads
    return {"ms": round(dt * 1e3, 2), "tflops": flops / dt / 1e12, "threads": 1,
            "sample": "tiny (32x32 grid, fp32, 1 head): pool + attention of all 1024 queries"}


def cpu_baseline(w, inp, shift, target_s: float):
    """The oracle, as it is, on a bounded sample of the same block: pooled K/V
    of all heads, then attention for R sampled query rows (R grown until one
    attention pass takes about target_s seconds; that pass is the value)."""
    import numpy as np

    from oracle import oracle as O

    p = O.Params(w.batch, w.heads, w.head_dim, w.grid, w.window, shift, w.pool, w.topk,
                 radius=w.radius, global_tokens=w.text)
    q, k, v = inp.f32("q"), inp.f32("k"), inp.f32("v")
    t0 = time.perf_counter()
    kp = O.global_rows(p, k, inp.f32("gk") if w.text else None)
    vp = O.global_rows(p, v, inp.f32("gv") if w.text else None)
    rt = O.route(p, q, k) if p.topk > 0 else None
    t_prep = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    total = w.batch * w.heads * w.n_tokens
    rows, t_att = 256, 0.0
    for _ in range(4):  # grow the sample until it takes about target_s
        sel = np.sort(rng.choice(total, size=rows, replace=False))
        t0 = time.perf_counter()
        O.attend_rows(p, q, k, v, sel, kp, vp, rt)
        t_att = time.perf_counter() - t0
        if t_att >= 0.5 * target_s or rows == total:
            break
        rows = int(min(total, rows * min(64.0, target_s / max(t_att, 1e-3))))
    flops = 4.0 * w.head_dim * p.keys_per_query * sel.size
    cores = O.num_threads()
    tiny = tiny_one_thread(O)
    O.set_num_threads(cores)
    return {
        "value": flops / t_att / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "tiny_1thread": tiny,
        "kind": "oracle",
        "sample": (f"{w.name} odd-shift block: float64 C oracle, pool{'+route' if rt is not None else ''}"
                   f" of all {w.heads} heads ({t_prep:.2f} s, not in value) then attention for "
                   f"{sel.size} sampled query rows x {p.keys_per_query} keys ({t_att:.2f} s); "
                   f"value = 4*d*L*rows / attention time"),
    }


class Workbench:
    """Plans, blocks and resident inputs of one workload, and the timings the
    JSON line reports for it.  Every time is taken with HIP events recorded
    on the stream the kernels run on (torch's current stream)."""

    def __init__(self, torch, basa, w):
        from video_gen_amd.synth import make_inputs

        self.torch, self.basa, self.w = torch, basa, w
        t0 = time.perf_counter()
        self.inp = make_inputs(w)
        self.q, self.k, self.v = (self.inp.torch(n) for n in ("q", "k", "v"))
        log(f"[bench] {w.name}: inputs ready in {time.perf_counter() - t0:.1f} s")
        self.blocks = [self.block(self.plan((0, 0, 0))), self.block(self.plan(w.shift))]
        self.stream = torch.cuda.current_stream()

    def plan(self, shift, dense=False):
        w, basa = self.w, self.basa
        # Extra global rows (text tokens) are keys of every query, dense too.
        if dense:
            return basa.Plan(w.batch, w.heads, w.head_dim, w.grid, w.grid, (0, 0, 0), (0, 0, 0),
                             0, w.dtype, global_tokens=w.text)
        return basa.Plan(w.batch, w.heads, w.head_dim, w.grid, w.window, shift, w.pool, w.topk,
                         w.dtype, route_radius=w.radius, global_tokens=w.text)

    def block(self, pl):
        b = self.basa.Block(pl)
        if self.w.text:
            b.set_global(self.inp.torch("gk"), self.inp.torch("gv"))
        return b

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def prepare(self, b):
        """Pooling and routing of one block (the kernels before attention)."""
        basa = self.basa
        if b.plan.info["pooled_tokens"]:
            basa.basa_pool_kv(b.plan, self.k, self.v, b.k_pool, b.v_pool)
        if b.route is not None:
            basa.basa_route_windows(b.plan, self.q, self.k, b.route, b.workspace)

    def attend(self, b):
        self.basa.basa_window_attn_fwd(b.plan, self.q, self.k, self.v, b.k_pool, b.v_pool,
                                       b.route, b.out)

    def steps(self, n_steps, n_warmup):
        """Times n_steps steps (both blocks: pool -> [route] -> attention);
        returns (ms per step, attention launch times in ms).  The step time
        comes from a pass with events only around the whole run; the
        per-launch attention times from a second pass of n_steps steps with
        events around each attention launch (each event is a packet of its
        own on the stream, so the first pass carries none)."""
        torch = self.torch
        ev = [(self.event(), self.event()) for _ in range(2 * n_steps)]

        def step(record=None):
            for i, b in enumerate(self.blocks):
                self.prepare(b)
                if record is not None:
                    record[i][0].record(self.stream)
                self.attend(b)
                if record is not None:
                    record[i][1].record(self.stream)

        for _ in range(n_warmup):
            step()
        torch.cuda.synchronize()
        start, stop = self.event(), self.event()
        start.record(self.stream)
        for _ in range(n_steps):
            step()
        stop.record(self.stream)
        torch.cuda.synchronize()
        for s in range(n_steps):
            step(ev[2 * s:2 * s + 2])
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n_steps, [a.elapsed_time(b) for a, b in ev]

    def attn_only_ms(self, n_steps):
        """Average attention launch over n_steps back-to-back pairs of the
        blocks' attention launches (even, odd), one event pair around all."""
        for b in self.blocks:
            self.attend(b)
        e0, e1 = self.event(), self.event()
        e0.record(self.stream)
        for _ in range(n_steps):
            for b in self.blocks:
                self.attend(b)
        e1.record(self.stream)
        self.torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n_steps * len(self.blocks))

    def prepare_ms(self, reps=20):
        """Pool + route of the odd block alone (0 if it does neither)."""
        b = self.blocks[1]
        if not b.plan.info["pooled_tokens"] and b.route is None:
            return 0.0
        e0, e1 = self.event(), self.event()
        e0.record(self.stream)
        for _ in range(reps):
            self.prepare(b)
        e1.record(self.stream)
        self.torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def exact_flops(self, b) -> float:
        """FLOPs of one attention launch of block b, the routed windows counted
        at their real sizes (from the route table its last routing wrote)."""
        if b.route is None:
            return b.plan.info["flops_sparse"]
        return self.basa.plan_pairs(b.plan, b.route.cpu().numpy())[1]

    def dense_ms(self, reps):
        """The same kernel with window = grid, no pooling, no routing."""
        dplan = self.plan(None, dense=True)
        dblk = self.block(dplan)
        dout = self.torch.empty_like(self.q)
        run = lambda: self.basa.basa_window_attn_fwd(dplan, self.q, self.k, self.v, dblk.k_pool,
                                                     dblk.v_pool, None, dout)
        for _ in range(2):
            run()
        self.torch.cuda.synchronize()
        d0, d1 = self.event(), self.event()
        d0.record(self.stream)
        for _ in range(reps):
            run()
        d1.record(self.stream)
        self.torch.cuda.synchronize()
        return d0.elapsed_time(d1) / reps, dplan.info["flops_sparse"]


def route_hbm(wb, reps=20):
    """Routing of the odd block alone: ms and GB/s for its HBM reads (Q and K
    once), or None if the workload does not route."""
    b = wb.blocks[1]
    if b.route is None:
        return None
    basa = wb.basa
    run = lambda: basa.basa_route_windows(b.plan, wb.q, wb.k, b.route, b.workspace)
    run()
    e0, e1 = wb.event(), wb.event()
    e0.record(wb.stream)
    for _ in range(reps):
        run()
    e1.record(wb.stream)
    wb.torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * wb.q.numel() * wb.q.element_size()
    return {"ms": round(ms, 4), "gbps_qk_read": round(nbytes / (ms / 1e3) / 1e9, 1)}


def flushed_attn_ms(wb, reps=10):
    """Median attention launch of the odd block with the caches emptied
    first: before each launch a 512 MB fill evicts L2 and the 256 MB
    last-level cache, so Q, K and V come from HBM."""
    torch = wb.torch
    junk = torch.empty(512 << 20, dtype=torch.uint8, device=wb.q.device)
    b = wb.blocks[1]
    wb.prepare(b)
    evs = []
    for _ in range(reps):
        junk.zero_()
        e0, e1 = wb.event(), wb.event()
        e0.record(wb.stream)
        wb.attend(b)
        e1.record(wb.stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del junk
    return statistics.median(a.elapsed_time(z) for a, z in evs)


def device_info():
    """CU count and maximum clock of the GPU agent from rocminfo, and the
    nominal dense bf16 rate they give (4096 flop per clock per CU).  Run
    before the process touches the GPU; None if rocminfo is not there."""
    import re
    import subprocess

    try:
        text = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in text.split("Agent ")[1:]:
        if not re.search(r"Name:\s+gfx", agent):
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        name = re.search(r"Name:\s+(gfx\w+)", agent)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return {"arch": name.group(1), "compute_units": cus, "max_clock_mhz": clk,
                    "nominal_bf16_tflops": round(cus * 4096 * clk * 1e6 / 1e12, 1)}
    return None


def mfma_probe(torch, basa, stream, mode, n_wg=512, iters=40000, reps=3):
    """The bf16 matrix-core rate this GPU sustains (libbasa's probe: two
    workgroups per CU, four product chains per wave; mode 0 constant
    operands, mode 1 operands whose bits switch from product to product) and
    its clock under that load, from the shader and 100 MHz clocks each
    workgroup read."""
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    clocks = torch.empty((n_wg, 4), dtype=torch.int64, device="cuda")
    basa.basa_probe_mfma(2000, n_wg, sink, clocks, mode=mode)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flops = basa.basa_probe_mfma(iters, n_wg, sink, clocks, mode=mode)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = clocks.cpu().numpy().astype(np.float64)
        ghz = float(np.median((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9))
        tflops = flops / (ms / 1e3) / 1e12
        if best is None or tflops > best["tflops"]:
            best = {"tflops": round(tflops, 1), "ms": round(ms, 3), "clock_ghz": round(ghz, 3)}
    ok = bool((sink == (4 * iters / 256.0 if mode == 0 else 0.0)).all().item())
    best.update({"workgroups": n_wg, "iters": iters, "sink_exact": ok})
    return best


def forward_summary(wb, metrics, n_steps, n_warmup, dense_reps):
    """Step time, attention time and its roofline fraction, dense speedup and
    kernel efficiency of one workload (both blocks, exact FLOPs)."""
    ms_step, attn_ms = wb.steps(n_steps, n_warmup)
    # The average launch: the steps' attention launches (both blocks, the
    # pooled rows and routes the steps left) issued back to back between one
    # event pair, as the dense run is timed.  Events around each launch add
    # their own packets to every launch (2-5 us at flux2k); the per-launch
    # times above give only the per-shift median and minimum.
    attn_avg = wb.attn_only_ms(n_steps)
    pre_ms = wb.prepare_ms()
    f_blocks = [wb.exact_flops(b) for b in wb.blocks]
    f_sparse = sum(f_blocks) / 2
    peak = metrics.MI355X_BF16_PEAK
    attn_tflops = f_sparse / (attn_avg / 1e3) / 1e12
    out = {
        "ms_per_step": ms_step,
        "step_tflops": sum(f_blocks) / (ms_step / 1e3) / 1e12,
        "attn_ms": attn_avg,
        "attn_by_shift": {name: {"median_ms": statistics.median(ts), "min_ms": min(ts)}
                          for name, ts in (("even", attn_ms[0::2]), ("odd", attn_ms[1::2]))},
        "attn_tflops": attn_tflops,
        "attn_frac_bf16_peak": attn_tflops * 1e12 / peak,
        "pool_route_ms": pre_ms,
        "flops_per_block": f_blocks,
        "dense_attn_ms": None, "dense_tflops": None, "speedup_measured": None,
        "speedup_theoretical": None, "kernel_eff": None, "kernel_eff_with_pool_route": None,
    }
    if dense_reps > 0:
        d_ms, f_dense = wb.dense_ms(dense_reps)
        out.update({
            "dense_attn_ms": d_ms,
            "dense_tflops": f_dense / (d_ms / 1e3) / 1e12,
            "speedup_measured": d_ms / attn_avg,
            "speedup_theoretical": f_dense / f_sparse,
            "kernel_eff": metrics.kernel_efficiency(d_ms, attn_avg, f_dense, f_sparse),
            "kernel_eff_with_pool_route": metrics.kernel_efficiency(d_ms, attn_avg + pre_ms,
                                                                    f_dense, f_sparse),
        })
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(BASA heads are independent; multi-GPU sharding is not part of this build)",
              file=sys.stderr)
        sys.exit(2)
    dev_info = device_info()
    import torch

    from video_gen_amd import basa, metrics
    from video_gen_amd.synth import WORKLOADS, make_grad

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    basa.load()
    w = WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: {w.description}")
    wb = Workbench(torch, basa, w)
    q, k, v, inp, blocks, stream = wb.q, wb.k, wb.v, wb.inp, wb.blocks, wb.stream
    info = blocks[0].plan.info
    fs = forward_summary(wb, metrics, args.steps, args.warmup, args.dense_reps)
    flushed_ms = flushed_attn_ms(wb, args.flush_reps) if args.flush_reps > 0 else None
    attn_avg = fs["attn_ms"]
    log(f"[bench] timed {args.steps} steps: {fs['ms_per_step']:.4f} ms/step, attention launch "
        f"avg {attn_avg:.4f} ms ({fs['attn_tflops']:.1f} TFLOP/s), dense "
        f"{fs['dense_attn_ms']} ms")

    # HBM-bound kernels on their own: the shift-aware gather (a windowed copy
    # of K, a plain copy of known size) and the K/V pooling.
    hbm = {}
    g_plan = blocks[1].plan
    xw = torch.empty((w.batch, w.heads, info["n_windows"], info["window_tokens"], w.head_dim),
                     dtype=k.dtype, device=k.device)
    elem = k.element_size()
    for _ in range(2):
        basa.basa_gather_windows(g_plan, k, xw)
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0.record(stream)
    for _ in range(20):
        basa.basa_gather_windows(g_plan, k, xw)
    h1.record(stream)
    torch.cuda.synchronize()
    g_ms = h0.elapsed_time(h1) / 20
    g_bytes = 2 * k.numel() * elem
    hbm["gather_ms"] = round(g_ms, 4)
    hbm["gather_gbps"] = round(g_bytes / (g_ms / 1e3) / 1e9, 1)
    del xw
    if blocks[1].plan.info["pooled_tokens"]:
        b = blocks[1]
        h0.record(stream)
        for _ in range(20):
            basa.basa_pool_kv(b.plan, k, v, b.k_pool, b.v_pool)
        h1.record(stream)
        torch.cuda.synchronize()
        p_ms = h0.elapsed_time(h1) / 20
        p_bytes = (2 * k.numel() + 2 * k.numel() // w.n_tokens * b.plan.info["pooled_tokens"]) * elem
        hbm["pool_ms"] = round(p_ms, 4)
        hbm["pool_gbps"] = round(p_bytes / (p_ms / 1e3) / 1e9, 1)
    if blocks[1].route is not None:
        hbm["route"] = route_hbm(wb)
    log(f"[bench] HBM kernels: {hbm}")

    # Backward of the odd block's attention (recomputes P from the forward's
    # lse; dO is a seeded standard-normal tensor).  Algorithmic work: the five
    # products of attention's backward, 2.5x the forward's FLOPs; the kernels
    # run seven (S and dP once for dq, once for the key gradients).
    bwd = None
    if args.bwd_reps > 0:
        b = blocks[1]
        lse = torch.empty(b.plan.token_shape[:3], dtype=torch.float32, device=q.device)
        g = make_grad(w)
        d_out = (torch.from_numpy(g.view("int16")).to(q.device).view(torch.bfloat16)
                 if w.dtype == "bf16" else torch.from_numpy(g).to(q.device))
        del g
        b.forward(q, k, v, lse)
        for _ in range(2):
            b.backward(q, k, v, lse, d_out)
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(args.bwd_reps):
            b.backward(q, k, v, lse, d_out)
        b1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / args.bwd_reps
        f_fwd = fs["flops_per_block"][1]
        f_bwd = 2.5 * f_fwd
        bwd = {
            "ms": round(bwd_ms, 4),
            "tflops": round(f_bwd / (bwd_ms / 1e3) / 1e12, 1),
            "frac_bf16_peak": round(f_bwd / (bwd_ms / 1e3) / metrics.MI355X_BF16_PEAK, 4),
            "mfma_tflops_executed": round(3.5 * f_fwd / (bwd_ms / 1e3) / 1e12, 1),
            "vs_forward": round(bwd_ms / attn_avg, 2),
            "reps": args.bwd_reps,
        }
        del d_out, lse
        log(f"[bench] attention backward: {bwd}")

    # The pages' own execution form: the key-list segments as separate
    # branches merged by log-sum-exp (two- and three-way), same block.
    split = None
    if args.bwd_reps > 0:
        b = blocks[1]
        ws = torch.empty(max(1, -(-b.plan.info["split_workspace_bytes"] // 8)),
                         dtype=torch.float64, device=q.device)
        split = {"fused_ms": round(attn_avg, 4)}
        for ways in (2, 3):
            for _ in range(2):
                basa.basa_window_attn_fwd_split(b.plan, q, k, v, b.k_pool, b.v_pool, b.route,
                                                b.out, None, ways, ws)
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(args.bwd_reps):
                basa.basa_window_attn_fwd_split(b.plan, q, k, v, b.k_pool, b.v_pool, b.route,
                                                b.out, None, ways, ws)
            s1.record(stream)
            torch.cuda.synchronize()
            split[f"split{ways}_ms"] = round(s0.elapsed_time(s1) / args.bwd_reps, 4)
        del ws
        log(f"[bench] branch-split forms: {split}")

    # Text queries of a joint block (workloads with text rows): dense over
    # every image token and text row, 4*d*X*(N+X) FLOPs per head.
    text = None
    if args.bwd_reps > 0 and w.text > 0:
        b = blocks[1]
        qt = torch.empty(b.plan.text_shape, dtype=q.dtype, device=q.device).normal_()
        for _ in range(2):
            b.text_forward(qt, k, v)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.bwd_reps):
            b.text_forward(qt, k, v)
        t1.record(stream)
        torch.cuda.synchronize()
        text_ms = t0.elapsed_time(t1) / args.bwd_reps
        f_text = 4.0 * w.head_dim * w.text * (w.n_tokens + w.text) * w.batch * w.heads
        text = {
            "ms": round(text_ms, 4),
            "tflops": round(f_text / (text_ms / 1e3) / 1e12, 1),
            "frac_bf16_peak": round(f_text / (text_ms / 1e3) / metrics.MI355X_BF16_PEAK, 4),
            "text_rows": w.text,
        }
        del qt
        log(f"[bench] text queries: {text}")

    # The video workload beside the main one, so that a Wan-shaped attention
    # figure (the pages' Table 3 row is attention-only latency after warm-up)
    # comes from the same run.
    video, video_more = None, []
    names = [n for n in args.video_workload.split(",") if n and n != "none" and n != w.name]
    for vname in names:
        vw = WORKLOADS[vname]
        log(f"[bench] video workload {vw.name}: {vw.description}")
        vb = Workbench(torch, basa, vw)
        vs = forward_summary(vb, metrics, max(5, args.steps // 2), max(2, args.warmup // 2),
                             max(2, args.dense_reps // 2))
        entry = {"workload": vw.name, "description": vw.description,
                 **{key: (_r(val, 4) if isinstance(val, float) else val)
                    for key, val in vs.items() if key != "flops_per_block"},
                 "gflop_per_block": [round(f / 1e9, 2) for f in vs["flops_per_block"]],
                 "route": route_hbm(vb)}
        entry["attn_by_shift"] = {k2: {k3: round(v3, 4) for k3, v3 in v2.items()}
                                  for k2, v2 in vs["attn_by_shift"].items()}
        log(f"[bench] video: {entry}")
        if video is None:
            video = entry
        else:
            video_more.append(entry)
        del vb

    # Last of the GPU work: the probe runs the matrix cores flat out.
    probe = None
    if not args.no_probe:
        probe = {"constant_operands": mfma_probe(torch, basa, stream, 0),
                 "switching_operands": mfma_probe(torch, basa, stream, 1)}
        log(f"[bench] MFMA probe: {probe}")
    peak = metrics.MI355X_BF16_PEAK
    traffic = measured_traffic(w.name)
    result = {
        "metric": METRIC,
        "value": round(fs["step_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fs["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "step": "even block (shift 0) + odd block (shift s), each pool -> "
                    + ("route -> " if w.topk else "") + "window attention",
            "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim, "tokens": w.n_tokens,
            "window_tokens": info["window_tokens"], "keys_per_query": info["keys_per_query"],
        },
        "attn_ms": round(attn_avg, 4),
        "attn_tflops": round(fs["attn_tflops"], 1),
        "attn_frac_bf16_peak": round(fs["attn_frac_bf16_peak"], 4),
        "attn_by_shift": {k2: {k3: round(v3, 4) for k3, v3 in v2.items()}
                          for k2, v2 in fs["attn_by_shift"].items()},
        "attn_flushed_ms": _r(flushed_ms, 4),
        "pool_route_ms": round(fs["pool_route_ms"], 4),
        "dense_attn_ms": _r(fs["dense_attn_ms"], 3),
        "dense_tflops": _r(fs["dense_tflops"], 1),
        "speedup_measured": _r(fs["speedup_measured"], 3),
        "speedup_theoretical": _r(fs["speedup_theoretical"], 3),
        "kernel_eff": _r(fs["kernel_eff"], 4),
        "kernel_eff_with_pool_route": _r(fs["kernel_eff_with_pool_route"], 4),
        "hbm_kernels": hbm,
        "backward": bwd,
        "branch_split": split,
        "text_queries": text,
        "video": video,
        "video_more": video_more,
        "roofline": {
            "bound": "mfma",
            "achieved": round(fs["attn_tflops"], 1),
            "peak": peak / 1e12,
            "unit": "TFLOP/s",
            "frac": round(fs["attn_frac_bf16_peak"], 4),
            "traffic": traffic,
        },
        "device": dev_info,
        "mfma_probe": probe,
        "attn_frac_of_probe": (round(fs["attn_tflops"] / probe["switching_operands"]["tflops"], 4)
                               if probe else None),
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        log("[bench] CPU oracle sample ...")
        result["cpu_baseline"] = cpu_baseline(w, inp, w.shift, args.cpu_seconds)
        log(f"[bench] CPU oracle: {result['cpu_baseline']['value']:.4f} TFLOP/s on "
            f"{result['cpu_baseline']['cores']} threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
