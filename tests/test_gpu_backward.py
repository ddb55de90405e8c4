"""GPU parity of the attention backward (basa_window_attn_bwd through the C
ABI) against the oracle's float64 gradients.

The GPU runs the five products on bf16 operands with float32 accumulation
and rounds P and dS to bf16 (and float32 inputs to bf16), so each gradient
is compared relative to its own scale, in units of bf16's unit roundoff
u = 2^-8: max |err| <= 2e-2 (~5u) * max |ref| and mean |err| <= 8e-3 (~2u) *
mean |ref|.  A gradient that is exactly zero (one-key lists have dS = 0)
gets an absolute floor of 1e-3 (max) and 1e-4 (mean).
Small problems are compared in full (every gradient, the global rows'
included).  Full-size workloads in the benchmark's launch configuration are
compared on sampled dq rows, on the token-key gradients of sampled windows
(both computed by the oracle from the queries involved alone), and on two
identities that hold at any size: over all keys the dV rows sum to the sum
of dO, and the dK rows sum to zero.
"""
import dataclasses

import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_util import basa_plan, oracle_params, sample_rows, say, to_f64
from video_gen_amd.synth import (WORKLOADS, Workload, bits_to_f32, make_grad, make_inputs,
                                 random_problem, random_short_problem)

pytestmark = pytest.mark.gpu

REL_MAX = 2e-2
REL_MEAN = 8e-3
# Sum of dV over all keys minus sum of dO, relative to sqrt(sum dO^2): each
# term is dO_n times the deviation of P_n's row sum from one (bf16 P), so
# the ratio is about the rms row-sum deviation.
IDENTITY_V = 1e-2
# Sum of dK over all keys, relative to sqrt(sum dK^2): each query adds
# scale q_n sum_j dS_nj, which is not exactly zero because delta = dO.O uses
# the bf16 forward output; at these shapes that is a few 1e-2 at most.
IDENTITY_K = 5e-2


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from video_gen_amd import basa

    basa.load()
    return torch, basa


def compare_grad(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = max(np.abs(ref).max(), 1e-3), max(np.abs(ref).mean(), 1e-4)
    say(f"  {what}: max_err/max_ref={err.max() / mx:.3e} mean_err/mean_ref={err.mean() / mean:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert err.max() <= REL_MAX * mx, f"{what}: max error {err.max():.3e} > {REL_MAX} * {mx:.3e}"
    assert err.mean() <= REL_MEAN * mean, f"{what}: mean error {err.mean():.3e} > {REL_MEAN} * {mean:.3e}"


def _dout_torch(torch, w, g):
    if w.dtype == "bf16":
        return torch.from_numpy(g.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(g).cuda()


def _gpu(torch, basa, plan, w, inp, g):
    blk = basa.Block(plan)
    if inp.gk is not None:
        blk.set_global(inp.torch("gk"), inp.torch("gv"))
    q, k, v = inp.torch("q"), inp.torch("k"), inp.torch("v")
    lse = torch.empty(plan.token_shape[:3], dtype=torch.float32, device="cuda")
    blk.forward(q, k, v, lse)
    grads = blk.backward(q, k, v, lse, _dout_torch(torch, w, g))
    torch.cuda.synchronize()
    return blk, [None if t is None else to_f64(t) for t in grads]


def _oracle_kv(w, p, inp):
    q, k, v = inp.f32("q"), inp.f32("k"), inp.f32("v")
    gk = inp.f32("gk") if inp.gk is not None else None
    gv = inp.f32("gv") if inp.gk is not None else None
    kp = O.global_rows(p, k, gk)
    vp = O.global_rows(p, v, gv)
    rt = O.route(p, q, k) if p.topk > 0 else None
    return q, k, v, kp, vp, rt


def _f32(w, g):
    return bits_to_f32(g) if w.dtype == "bf16" else g


def _full_check(torch, basa, w, shift, heads=None, tag=""):
    inp = make_inputs(w, heads=heads)
    g = make_grad(w, heads=heads)
    wl = w if heads is None else dataclasses.replace(w, heads=heads)
    plan = basa_plan(basa, wl, shift)
    blk, (dq, dk, dv, dkg, dvg) = _gpu(torch, basa, plan, wl, inp, g)
    p = oracle_params(wl, shift)
    q, k, v, kp, vp, rt = _oracle_kv(wl, p, inp)
    if rt is not None:
        np.testing.assert_array_equal(blk.route.cpu().numpy(), rt)
    ref = O.attend_bwd(p, q, k, v, _f32(w, g), kp, vp, rt)
    compare_grad(dq, ref["dq"], f"{tag} dq")
    compare_grad(dk, ref["dk"], f"{tag} dk")
    compare_grad(dv, ref["dv"], f"{tag} dv")
    if ref["dkg"] is not None:
        compare_grad(dkg, ref["dkg"], f"{tag} dk_global")
        compare_grad(dvg, ref["dvg"], f"{tag} dv_global")
    else:
        assert dkg is None and dvg is None


@pytest.mark.parametrize("name,heads", [("tiny", None), ("flux1k", 2), ("flux2k", 1)])
@pytest.mark.parametrize("odd", [False, True])
def test_bwd_full_small(env, name, heads, odd):
    torch, basa = env
    w = WORKLOADS[name]
    say(f"[bwd-full] {name} heads={heads} odd={odd}")
    _full_check(torch, basa, w, w.shift if odd else (0, 0, 0), heads, name)


def test_bwd_random_small_configs(env):
    """Random grids, windows, shifts, pools and routing (d = 64 and 128),
    one-token windows, window = grid, topk = nW - 1, a routing radius, short
    windows and extra global rows."""
    torch, basa = env
    rng = np.random.default_rng(1234)
    cases = []
    for _ in range(4):
        grid, window, shift, pool = random_problem(rng, max_tokens=400)
        nw = int(np.prod([-(-g // x) for g, x in zip(grid, window)]))
        topk = int(rng.integers(0, min(nw, 4))) if nw > 1 else 0
        cases.append((grid, window, shift, pool if rng.integers(0, 2) else (0, 0, 0), topk))
    cases.append(((1, 8, 8), (1, 1, 1), (0, 3, 5), (0, 0, 0), 0))        # one-token windows
    cases.append(((2, 8, 12), (2, 8, 12), (1, 2, 3), (2, 8, 12), 0))     # window = grid, G = 1
    cases.append(((1, 12, 12), (1, 4, 4), (0, 1, 1), (1, 3, 3), 8))      # topk = nW - 1
    cases.append(((3, 16, 16), (3, 4, 4), (0, 2, 1), (1, 4, 4), 3, 1))  # video, radius 1
    for _ in range(3):                                                   # short windows
        grid, window, shift, pool = random_short_problem(rng, max_tokens=400)
        nw = int(np.prod([-(-g // x) for g, x in zip(grid, window)]))
        topk = int(rng.integers(0, min(nw, 4))) if nw > 1 else 0
        cases.append((grid, window, shift, pool, topk))
    cases.append(((1, 16, 16), (1, 8, 8), (0, 4, 4), (1, 4, 4), 0, -1, 77))   # text rows
    cases.append(((2, 12, 12), (2, 4, 4), (1, 2, 2), (0, 0, 0), 2, -1, 300))  # text only
    # float32 plans (inputs rounded to bf16 copies): short windows with routing
    # and text rows, and a routed radius case
    cases.append(((2, 7, 10), (2, 3, 4), (1, 2, 3), (1, 7, 5), 2, -1, 5, "f32"))
    cases.append(((3, 16, 16), (3, 4, 4), (0, 2, 1), (1, 4, 4), 3, 1, 0, "f32"))
    for i, case in enumerate(cases):
        grid, window, shift, pool, topk = case[:5]
        radius = case[5] if len(case) > 5 else -1
        text = case[6] if len(case) > 6 else 0
        dtype = case[7] if len(case) > 7 else "bf16"
        d = 64 if i % 2 else 128
        wl = Workload("rand", 1, 2, d, grid, window, shift, pool, topk, dtype, 700 + i, True,
                      "random small", radius=radius, text=text)
        say(f"[bwd-rand] d={d} grid={grid} window={window} shift={shift} pool={pool} "
            f"topk={topk} radius={radius} text={text} dtype={dtype}")
        _full_check(torch, basa, wl, shift, tag=f"case {i}")


@pytest.mark.parametrize("name", ["flux2k", "flux2k_text", "flux4k", "wan", "wan_t3w10", "wan_t3"])
def test_bwd_sampled_full_size(env, name):
    torch, basa = env
    w = WORKLOADS[name]
    say(f"[bwd-sampled] {name}")
    inp = make_inputs(w)
    g = make_grad(w)
    plan = basa_plan(basa, w, w.shift)
    blk, (dq, dk, dv, dkg, dvg) = _gpu(torch, basa, plan, w, inp, g)
    p = oracle_params(w, w.shift)
    q, k, v, kp, vp, rt = _oracle_kv(w, p, inp)
    if rt is not None:
        np.testing.assert_array_equal(blk.route.cpu().numpy(), rt)
    _, _, tok = O.partition(oracle_params(w, w.shift, heads=1))
    rows = sample_rows(w, tok, w.heads, 2000, seed=41)
    ref = O.attend_bwd_dq_rows(p, q, k, v, _f32(w, g), rows, kp, vp, rt)
    compare_grad(dq.reshape(-1, w.head_dim)[rows], ref, f"{name} dq[{rows.size} rows]")
    # Identities over all keys: the extra global rows are keys too; the
    # pooled cells' share is already in dk, dv.
    G = plan.info["pooled_tokens"]
    sv = dv.sum(axis=2)
    sk = dk.sum(axis=2)
    if dvg is not None:
        sv += dvg[:, :, G:].sum(axis=2)
        sk += dkg[:, :, G:].sum(axis=2)
    want_v = _f32(w, g).astype(np.float64).sum(axis=2)
    gn = np.sqrt((_f32(w, g).astype(np.float64) ** 2).sum(axis=2))
    ev = (np.abs(sv - want_v) / gn).max()
    ek = (np.abs(sk) / np.sqrt((dk ** 2).sum(axis=2))).max()
    say(f"  {name} identities: |sum dV - sum dO| / |dO| {ev:.3e}, |sum dK| / |dK| {ek:.3e}")
    assert ev <= IDENTITY_V and ek <= IDENTITY_K
    if name in KEY_CHECK:
        _check_window_keys(w, p, plan, inp, g, dk, dv, dkg, dvg, tok, q, k, v, kp, vp, rt,
                           full=name not in ("wan_t3", "wan_t3w10"))


# Workloads whose sampled windows' key gradients are compared element-wise
# (every query of the window and of the windows routed to it enters them):
# two windows at the first and last head, or, for the long key lists of the
# Table 3 shapes, the last window (a short one at wan_t3w10) of the first
# head.
KEY_CHECK = ("flux2k", "flux2k_text", "flux4k", "wan", "wan_t3", "wan_t3w10")


def _cells(w):
    T, H, W = w.grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    pt, ph, pw = w.pool
    gy, gx = H // ph, W // pw
    return (((t // pt) * gy + y // ph) * gx + x // pw).reshape(-1)


def _check_window_keys(w, p, plan, inp, g, dk, dv, dkg, dvg, tok, q, k, v, kp, vp, rt,
                       full=True):
    nw = tok.shape[0]
    if full:
        bhs = (0, w.batch * w.heads - 1)
        wins = (nw - 1, int(np.random.default_rng(5).integers(0, nw)))
        pairs = [(bh, wi) for bh in bhs for wi in wins]
    else:
        pairs = [(0, nw - 1)]
    gf = _f32(w, g)
    # each oracle call runs its queries on every host thread
    refs = [O.attend_bwd_window_keys(p, q, k, v, gf, bh, wi, kp, vp, rt) for bh, wi in pairs]
    pooled = plan.info["pooled_tokens"] > 0
    cell = _cells(w) if pooled else None
    P = int(np.prod(w.pool)) if pooled else 1
    for (bh, wi), (rk, rv) in zip(pairs, refs):
        t = tok[wi][tok[wi] >= 0]
        b, h = divmod(bh, w.heads)
        gk_, gv_ = dk[b, h, t], dv[b, h, t]
        if pooled:
            gk_ = gk_ - dkg[b, h, cell[t]] / P
            gv_ = gv_ - dvg[b, h, cell[t]] / P
        compare_grad(gk_, rk[:t.size], f"dk of window {wi} at bh {bh}")
        compare_grad(gv_, rv[:t.size], f"dv of window {wi} at bh {bh}")


def test_bwd_rejects_bad_workspace(env):
    torch, basa = env
    w = WORKLOADS["tiny"]
    plan = basa_plan(basa, w, w.shift)
    inp = make_inputs(w)
    blk = basa.Block(plan)
    q, k, v = inp.torch("q"), inp.torch("k"), inp.torch("v")
    lse = torch.empty(plan.token_shape[:3], dtype=torch.float32, device="cuda")
    blk.forward(q, k, v, lse)
    f = lambda: torch.empty(plan.token_shape, dtype=torch.float32, device="cuda")  # noqa: E731
    gshape = plan.pooled_shape
    small = torch.empty(16, dtype=torch.float64, device="cuda")
    with pytest.raises(basa.BasaError):
        basa.basa_window_attn_bwd(plan, q, k, v, blk.k_pool, blk.v_pool, None, blk.out, lse, q,
                                  f(), f(), f(), torch.empty(gshape, device="cuda"),
                                  torch.empty(gshape, device="cuda"), small)
    torch.cuda.synchronize()
