"""Pins of the oracle's backward pass (CPU only).

The gradients of BASA attention (what the pages' sparse adaptation, sec. 3.4,
trains through) are pinned two ways that share nothing with the oracle's own
loops: central finite differences of its forward pass, and torch autograd (in
float64) through a dense masked formulation: K/V mean-pooled with torch
reshapes, the key mask built from the NumPy partition and the route table,
one softmax, one product.
"""
import math

import numpy as np
import pytest
import torch

from oracle import brute
from oracle.oracle import Params


def _problem(seed, grid=(1, 8, 8), window=(1, 4, 4), shift=(0, 1, 2), pool=(1, 2, 2), topk=1,
             X=3, d=8, heads=2):
    p = Params(1, heads, d, grid, window, shift, pool, topk, global_tokens=X)
    g = np.random.default_rng(seed)
    n = p.n_tokens
    f = lambda *s: g.standard_normal(s).astype(np.float32)  # noqa: E731
    return p, f(1, heads, n, d), f(1, heads, n, d), f(1, heads, n, d), f(1, heads, X, d), \
        f(1, heads, X, d), f(1, heads, n, d)


def _loss(oracle_lib, p, q, k, v, gk, gv, dout, rt):
    kp = oracle_lib.global_rows(p, k, gk)
    vp = oracle_lib.global_rows(p, v, gv)
    out, _ = oracle_lib.attend(p, q, k, v, kp, vp, rt)
    return float((out * dout.astype(np.float64)).sum())


def test_backward_matches_finite_differences(oracle_lib):
    p, q, k, v, gk, gv, dout = _problem(1)
    rt = oracle_lib.route(p, q, k)
    kp = oracle_lib.global_rows(p, k, gk)
    vp = oracle_lib.global_rows(p, v, gv)
    grads = oracle_lib.attend_bwd(p, q, k, v, dout, kp, vp, rt)
    G = p.pooled_tokens
    h = 2.0 ** -10                 # exact in float32 at these magnitudes
    rng = np.random.default_rng(7)
    arrays = dict(q=q, k=k, v=v, gk=gk, gv=gv)
    want = dict(q=grads["dq"], k=grads["dk"], v=grads["dv"], gk=grads["dkg"][:, :, G:],
                gv=grads["dvg"][:, :, G:])
    for name, arr in arrays.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            x0 = arr[idx]
            vals = []
            for sgn in (1.0, -1.0):
                arr[idx] = np.float32(x0 + sgn * h)
                vals.append(_loss(oracle_lib, p, q, k, v, gk, gv, dout, rt))
            arr[idx] = x0
            fd = (vals[0] - vals[1]) / (2 * h)
            # routing is fixed (a selection has no gradient): the perturbation
            # is far too small to change it here
            assert fd == pytest.approx(want[name][idx], rel=2e-4, abs=2e-6), (name, idx)


def _pool_t(x, grid, pool):
    B, H, N, d = x.shape
    T, Hg, Wg = grid
    pt, ph, pw = pool
    g = x.reshape(B, H, T // pt, pt, Hg // ph, ph, Wg // pw, pw, d)
    return g.mean(dim=(3, 5, 7)).reshape(B, H, -1, d)


@pytest.mark.parametrize("case", [
    dict(grid=(1, 8, 8), window=(1, 4, 4), shift=(0, 1, 2), pool=(1, 2, 2), topk=1, X=3),
    dict(grid=(2, 6, 8), window=(1, 3, 4), shift=(1, 2, 3), pool=(2, 3, 2), topk=2, X=0),
    dict(grid=(1, 10, 12), window=(1, 4, 5), shift=(0, 3, 1), pool=(0, 0, 0), topk=2, X=5),
])
def test_backward_matches_torch_autograd(oracle_lib, case):
    """Short windows included (the third case): the mask comes from the NumPy
    padded partition."""
    p, q, k, v, gk, gv, dout = _problem(11, **case)
    rt = oracle_lib.route(p, q, k) if p.topk else None
    kp = oracle_lib.global_rows(p, k, gk if p.global_tokens else None)
    vp = oracle_lib.global_rows(p, v, gv if p.global_tokens else None)
    got = oracle_lib.attend_bwd(p, q, k, v, dout, kp, vp, rt)

    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in dict(q=q, k=k, v=v, gk=gk, gv=gv).items()}
    kcols, vcols = [t["k"]], [t["v"]]
    if p.pool_on:
        kcols.append(_pool_t(t["k"], p.grid, p.pool))
        vcols.append(_pool_t(t["v"], p.grid, p.pool))
    if p.global_tokens:
        kcols.append(t["gk"])
        vcols.append(t["gv"])
    kk, vv = torch.cat(kcols, 2), torch.cat(vcols, 2)
    tok = brute.partition_tok(p.grid, p.window, p.shift)
    n_glob = kk.shape[2] - p.n_tokens
    mask = torch.from_numpy(brute.key_mask(tok, rt, p.n_tokens, n_glob))
    z = torch.einsum("bhnd,bhjd->bhnj", t["q"], kk) / math.sqrt(p.dim)
    z = torch.where(mask, z, torch.tensor(-math.inf, dtype=torch.float64))
    out = torch.einsum("bhnj,bhjd->bhnd", torch.softmax(z, -1), vv)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(got["dq"], t["q"].grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(got["dk"], t["k"].grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(got["dv"], t["v"].grad.numpy(), atol=1e-10, rtol=0)
    if p.global_tokens:
        G = p.pooled_tokens
        np.testing.assert_allclose(got["dkg"][:, :, G:], t["gk"].grad.numpy(), atol=1e-10, rtol=0)
        np.testing.assert_allclose(got["dvg"][:, :, G:], t["gv"].grad.numpy(), atol=1e-10, rtol=0)


def test_dq_rows_equal_full_backward(oracle_lib):
    """dq of a query depends on its own key list alone: the row variant gives
    the full backward's rows exactly (short windows, routing, text rows)."""
    p, q, k, v, gk, gv, dout = _problem(3, grid=(2, 7, 10), window=(2, 3, 4), shift=(1, 2, 3),
                                        pool=(1, 7, 5), topk=2, X=5)
    rt = oracle_lib.route(p, q, k)
    kp = oracle_lib.global_rows(p, k, gk)
    vp = oracle_lib.global_rows(p, v, gv)
    full = oracle_lib.attend_bwd(p, q, k, v, dout, kp, vp, rt)["dq"].reshape(-1, p.dim)
    rows = np.array([0, 5, 77, 139, 140, 200, 279], np.int64)
    got = oracle_lib.attend_bwd_dq_rows(p, q, k, v, dout, rows, kp, vp, rt)
    np.testing.assert_array_equal(got, full[rows])


@pytest.mark.parametrize("case", [dict(), dict(grid=(2, 7, 10), window=(2, 3, 4), shift=(1, 2, 3),
                                           pool=(1, 7, 5), topk=2, X=5)])
def test_backward_sum_identities(oracle_lib, case):
    """Each softmax row sums to one, so over all keys (tokens after the pooled
    share is carried back, plus the extra global rows) the dV rows add up to
    the sum of dO and the dK rows add up to zero."""
    p, q, k, v, gk, gv, dout = _problem(4, **case)
    rt = oracle_lib.route(p, q, k)
    kp = oracle_lib.global_rows(p, k, gk)
    vp = oracle_lib.global_rows(p, v, gv)
    g = oracle_lib.attend_bwd(p, q, k, v, dout, kp, vp, rt)
    G = p.pooled_tokens
    sv = g["dv"].sum(axis=2) + g["dvg"][:, :, G:].sum(axis=2)
    sk = g["dk"].sum(axis=2) + g["dkg"][:, :, G:].sum(axis=2)
    np.testing.assert_allclose(sv, dout.astype(np.float64).sum(axis=2), rtol=0, atol=1e-10)
    np.testing.assert_allclose(sk, 0.0, rtol=0, atol=1e-10)


def _cell_of_tokens(grid, pool):
    T, H, W = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    gy, gx = H // pool[1], W // pool[2]
    return (((t // pool[0]) * gy + y // pool[1]) * gx + x // pool[2]).reshape(-1)


def test_window_keys_equal_full_backward(oracle_lib):
    """The per-window key gradients plus the pooled cells' share are the full
    backward's dk, dv rows of that window's tokens (short windows, routing,
    text rows)."""
    p, q, k, v, gk, gv, dout = _problem(5, grid=(2, 7, 10), window=(2, 3, 4), shift=(1, 2, 3),
                                        pool=(1, 7, 5), topk=2, X=5)
    rt = oracle_lib.route(p, q, k)
    kp = oracle_lib.global_rows(p, k, gk)
    vp = oracle_lib.global_rows(p, v, gv)
    full = oracle_lib.attend_bwd(p, q, k, v, dout, kp, vp, rt)
    _, _, tok = oracle_lib.partition(p)
    cell = _cell_of_tokens(p.grid, p.pool)
    P = int(np.prod(p.pool))
    for bh in (0, 1):
        for w in range(p.n_windows):
            dk, dv = oracle_lib.attend_bwd_window_keys(p, q, k, v, dout, bh, w, kp, vp, rt)
            t = tok[w][tok[w] >= 0]
            m = t.size
            np.testing.assert_allclose(dk[:m] + full["dkg"][0, bh, cell[t]] / P,
                                       full["dk"][0, bh, t], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dv[:m] + full["dvg"][0, bh, cell[t]] / P,
                                       full["dv"][0, bh, t], rtol=1e-12, atol=1e-12)
            assert not dk[m:].any() and not dv[m:].any()
