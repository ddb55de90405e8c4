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

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

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
    return {
        "value": flops / t_att / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": (f"{w.name} odd-shift block: float64 C oracle, pool{'+route' if rt is not None else ''}"
                   f" of all {w.heads} heads ({t_prep:.2f} s, not in value) then attention for "
                   f"{sel.size} sampled query rows x {p.keys_per_query} keys ({t_att:.2f} s); "
                   f"value = 4*d*L*rows / attention time"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(BASA heads are independent; multi-GPU sharding is not part of this build)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from video_gen_amd import basa, metrics
    from video_gen_amd.synth import WORKLOADS, make_grad, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    basa.load()
    w = WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: {w.description}")
    t0 = time.perf_counter()
    inp = make_inputs(w)
    q, k, v = inp.torch("q"), inp.torch("k"), inp.torch("v")
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    def plan(shift, dense=False):
        # Extra global rows (text tokens) are keys of every query, dense too.
        if dense:
            return basa.Plan(w.batch, w.heads, w.head_dim, w.grid, w.grid, (0, 0, 0), (0, 0, 0),
                             0, w.dtype, global_tokens=w.text)
        return basa.Plan(w.batch, w.heads, w.head_dim, w.grid, w.window, shift, w.pool, w.topk,
                         w.dtype, route_radius=w.radius, global_tokens=w.text)

    def block(pl):
        b = basa.Block(pl)
        if w.text:
            b.set_global(inp.torch("gk"), inp.torch("gv"))
        return b

    blocks = [block(plan((0, 0, 0))), block(plan(w.shift))]
    info = blocks[0].plan.info
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(2 * args.steps)]

    def step(record=None):
        for i, b in enumerate(blocks):
            if b.plan.info["pooled_tokens"]:
                basa.basa_pool_kv(b.plan, k, v, b.k_pool, b.v_pool)
            if b.route is not None:
                basa.basa_route_windows(b.plan, q, k, b.route, b.workspace)
            if record is not None:
                record[i][0].record(stream)
            basa.basa_window_attn_fwd(b.plan, q, k, v, b.k_pool, b.v_pool, b.route, b.out)
            if record is not None:
                record[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        step(ev[2 * s:2 * s + 2])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    ms_step = total_ms / args.steps
    attn_avg = sum(attn_ms) / len(attn_ms)
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step, attention launch avg "
        f"{attn_avg:.4f} ms")

    # Pool and route alone (same stream, HIP events), for the breakdown.
    pre_ms = 0.0
    b = blocks[1]
    if b.plan.info["pooled_tokens"] or b.route is not None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record(stream)
        for _ in range(reps):
            if b.plan.info["pooled_tokens"]:
                basa.basa_pool_kv(b.plan, k, v, b.k_pool, b.v_pool)
            if b.route is not None:
                basa.basa_route_windows(b.plan, q, k, b.route, b.workspace)
        e1.record(stream)
        torch.cuda.synchronize()
        pre_ms = e0.elapsed_time(e1) / reps

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
        f_bwd = 2.5 * b.plan.info["flops_sparse"]
        bwd = {
            "ms": round(bwd_ms, 4),
            "tflops": round(f_bwd / (bwd_ms / 1e3) / 1e12, 1),
            "frac_bf16_peak": round(f_bwd / (bwd_ms / 1e3) / metrics.MI355X_BF16_PEAK, 4),
            "mfma_tflops_executed": round(3.5 * b.plan.info["flops_sparse"] / (bwd_ms / 1e3) / 1e12, 1),
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

    # Dense run of the same kernel (window = grid); --dense-reps 0 skips it.
    dense_ms = None
    dplan = plan(None, dense=True)
    if args.dense_reps > 0:
        dblk = block(dplan)
        dout = torch.empty_like(q)
        for _ in range(2):
            basa.basa_window_attn_fwd(dplan, q, k, v, dblk.k_pool, dblk.v_pool, None, dout)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.dense_reps):
            basa.basa_window_attn_fwd(dplan, q, k, v, dblk.k_pool, dblk.v_pool, None, dout)
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / args.dense_reps
        log(f"[bench] dense attention: {dense_ms:.3f} ms")

    # Dense work: full attention over the grid (plus any extra global rows).
    f_sparse, f_dense = info["flops_sparse"], dplan.info["flops_sparse"]
    peak = metrics.MI355X_BF16_PEAK
    attn_tflops = f_sparse / (attn_avg / 1e3) / 1e12
    step_tflops = 2 * f_sparse / (ms_step / 1e3) / 1e12
    theo = f_dense / f_sparse
    eff_attn = eff_block = None
    if dense_ms is not None:
        eff_attn = metrics.kernel_efficiency(dense_ms, attn_avg, f_dense, f_sparse)
        eff_block = metrics.kernel_efficiency(dense_ms, attn_avg + pre_ms, f_dense, f_sparse)
    traffic = measured_traffic(w.name)
    result = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
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
        "attn_tflops": round(attn_tflops, 1),
        "attn_frac_bf16_peak": round(attn_tflops * 1e12 / peak, 4),
        "pool_route_ms": round(pre_ms, 4),
        "dense_attn_ms": _r(dense_ms, 3),
        "dense_tflops": _r(dense_ms and f_dense / (dense_ms / 1e3) / 1e12, 1),
        "speedup_measured": _r(dense_ms and dense_ms / attn_avg, 3),
        "speedup_theoretical": round(theo, 3),
        "kernel_eff": _r(eff_attn, 4),
        "kernel_eff_with_pool_route": _r(eff_block, 4),
        "hbm_kernels": hbm,
        "backward": bwd,
        "branch_split": split,
        "text_queries": text,
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 1),
            "peak": peak / 1e12,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops * 1e12 / peak, 4),
            "traffic": traffic,
        },
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
