"""Brute-force formulations that pin the CPU oracle (TEST INFRASTRUCTURE ONLY).

Each function here computes the same quantity as an oracle function, but by a
different route, so that a dropped term, a wrong sign or index, or a transposed
operand in either one shows up as a disagreement:

* the window partition by the recipe the paperlayer.ai summary gives for BASA
  (A.1): cyclic shift of the grid, reshape, permute -- applied to an array of
  token indices with numpy's roll/reshape/transpose;
* average pooling by reshaping the grid into cells and taking numpy's mean;
* routing by a dense float64 score matrix and a stable argsort;
* attention as dense attention over [K ; pooled K] with an explicit
  N x (N + G) boolean mask (same window, a routed window, or a pooled cell),
  softmax and a matrix product -- the definition of "one softmax over the
  concatenated K/V tokens" (A.1) without any window bookkeeping.

Only small grids are meant here (the mask is dense).
"""
from __future__ import annotations

import numpy as np


def partition_tok(grid, window, shift) -> np.ndarray:
    """tok[w, s] by roll(-shift) + reshape + permute of the token-index grid.

    A grid a window does not divide is padded at the end of every axis with
    -1 (not a token) up to a window multiple before the reshape; each
    window's real tokens are then listed first, in their order, and its -1
    entries last."""
    T, H, W = grid
    wt, wh, ww = window
    idx = np.arange(T * H * W, dtype=np.int64).reshape(T, H, W)
    rolled = np.roll(idx, shift=(-shift[0], -shift[1], -shift[2]), axis=(0, 1, 2))
    pads = [(0, (-g) % w) for g, w in zip(grid, window)]
    rolled = np.pad(rolled, pads, constant_values=-1)
    nt, ny, nx = (rolled.shape[0] // wt, rolled.shape[1] // wh, rolled.shape[2] // ww)
    blocks = rolled.reshape(nt, wt, ny, wh, nx, ww).transpose(0, 2, 4, 1, 3, 5)
    tok = blocks.reshape(nt * ny * nx, wt * wh * ww)
    out = np.full_like(tok, -1)
    for w in range(tok.shape[0]):
        real = tok[w][tok[w] >= 0]
        out[w, :real.size] = real
    return out


def pool_mean(x: np.ndarray, grid, pool) -> np.ndarray:
    """[B, H, N, d] -> [B, H, G, d] by reshaping into cells and averaging."""
    B, Hh, N, d = x.shape
    T, H, W = grid
    pt, ph, pw = pool
    g = x.astype(np.float64).reshape(B, Hh, T // pt, pt, H // ph, ph, W // pw, pw, d)
    m = g.mean(axis=(3, 5, 7))
    return m.reshape(B, Hh, -1, d)


def route_topk(q: np.ndarray, k: np.ndarray, tok: np.ndarray, topk: int, wgrid=None,
               radius: int = -1):
    """Top-k windows by window-mean(q) . window-mean(k), excluding self and,
    for radius >= 0, every window whose (t, y, x) position in the window grid
    `wgrid` (from numpy's unravel_index) is more than `radius` away on an axis.

    Returns (route [B, H, nW, topk], margin [B, H, nW]) where margin is the
    relative gap between the k-th and (k+1)-th candidate score: rows whose
    margin is tiny are near-ties, where float64 rounding order may decide.
    """
    real = (tok >= 0)[None, None, :, :, None]            # short windows: -1 = no token
    safe = np.where(tok >= 0, tok, 0)
    qw = np.where(real, q.astype(np.float64)[:, :, safe, :], 0.0).mean(axis=3)  # [B, H, nW, d]
    kw = np.where(real, k.astype(np.float64)[:, :, safe, :], 0.0).mean(axis=3)
    sc = np.einsum("bhid,bhjd->bhij", qw, kw)
    B, Hh, nw, _ = sc.shape
    if radius >= 0:
        pos = np.stack(np.unravel_index(np.arange(nw), tuple(wgrid)), axis=1)  # [nW, 3]
        near = (np.abs(pos[:, None, :] - pos[None, :, :]) <= radius).all(axis=2)
    route = np.empty((B, Hh, nw, topk), np.int64)
    margin = np.full((B, Hh, nw), np.inf)
    for b in range(B):
        for h in range(Hh):
            for i in range(nw):
                cand = [j for j in range(nw) if j != i and (radius < 0 or near[i, j])]
                s = sc[b, h, i, cand]
                order = np.lexsort((np.array(cand), -s))  # score desc, then j asc
                route[b, h, i] = np.array(cand)[order[:topk]]
                if len(cand) > topk:
                    a, c = s[order[topk - 1]], s[order[topk]]
                    margin[b, h, i] = abs(a - c) / max(abs(a), abs(c), 1e-300)
    return route, margin


def key_mask(tok: np.ndarray, route, n_tokens: int, n_pooled: int) -> np.ndarray:
    """Boolean [B, H, N, N + G]: may query n attend to key column j?"""
    nw, m = tok.shape
    win_of = np.empty(n_tokens, np.int64)
    flat = tok.reshape(-1)
    win_of[flat[flat >= 0]] = np.repeat(np.arange(nw), m)[flat >= 0]
    same = win_of[:, None] == win_of[None, :]
    if route is None:
        allowed = same[None, None]
    else:
        B, Hh = route.shape[:2]
        allowed = np.empty((B, Hh, n_tokens, n_tokens), bool)
        for b in range(B):
            for h in range(Hh):
                routed = np.zeros((nw, nw), bool)
                for i in range(nw):
                    routed[i, route[b, h, i]] = True
                allowed[b, h] = same | routed[win_of[:, None], win_of[None, :]]
    pooled = np.ones(allowed.shape[:3] + (n_pooled,), bool)
    return np.concatenate([allowed, pooled], axis=-1)


def masked_attention(q, k, v, kp, vp, mask, scale):
    """Dense masked attention in float64: returns (out [B,H,N,d], lse [B,H,N])."""
    q = q.astype(np.float64)
    kk = k.astype(np.float64)
    vv = v.astype(np.float64)
    if kp is not None and kp.shape[2] > 0:
        kk = np.concatenate([kk, kp.astype(np.float64)], axis=2)
        vv = np.concatenate([vv, vp.astype(np.float64)], axis=2)
    z = scale * np.einsum("bhnd,bhjd->bhnj", q, kk)
    mask = np.broadcast_to(mask, z.shape)
    z = np.where(mask, z, -np.inf)
    zmax = z.max(axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    l = e.sum(axis=-1, keepdims=True)
    out = np.einsum("bhnj,bhjd->bhnd", e / l, vv)
    lse = (zmax + np.log(l))[..., 0]
    return out, lse


def exact_window_sums(x: np.ndarray, tok: np.ndarray):
    """Exact float64 window sums of routing, [BH, nW, d], of x [BH, N, d]
    (float32 values; tok [nW, M] with -1 past a short window's slots).

    The values are scaled by a power of two to integers and summed in int64,
    so no rounding happens before the final conversion; `exact` [BH, nW, d]
    is True where that exact sum is a float64 (then every summation order in
    float64 gives the same bits, since no partial sum can round: each is a
    multiple of the same quantum, smaller than 2^53 quanta).  Needs the
    exponent span of x plus log2(M) to fit int64; raises otherwise."""
    bh, n, d = x.shape
    bits = np.ascontiguousarray(x, np.float32).view(np.uint32)
    sig = 8 if not (bits & 0xFFFF).any() else 24      # bfloat16 values: 8 significant bits
    v = x.astype(np.float64)
    nz = v[v != 0]
    if nz.size == 0:
        return np.zeros((bh, tok.shape[0], d)), np.ones((bh, tok.shape[0], d), bool)
    e = np.frexp(nz)[1]
    emin, emax = int(e.min()) - sig, int(e.max())
    m = tok.shape[1]
    if emax - emin + int(np.ceil(np.log2(max(m, 2)))) + 1 > 62:
        raise ValueError("exponent span too wide for an int64 sum")
    scaled = np.ldexp(v, -emin)
    ints = scaled.astype(np.int64)
    assert (ints.astype(np.float64) == scaled).all(), "scaling did not give integers"
    real = tok >= 0
    safe = np.where(real, tok, 0)
    sums = np.empty((bh, tok.shape[0], d))
    exact = np.empty((bh, tok.shape[0], d), bool)
    for b in range(bh):
        s = (ints[b][safe] * real[:, :, None]).sum(axis=1)      # int64, exact
        f = s.astype(np.float64)
        exact[b] = f.astype(np.int64) == s       # |s| < 2^62: the conversion back is safe
        sums[b] = np.ldexp(f, emin)
    return sums, exact


def fsum_window_sums(x: np.ndarray, tok: np.ndarray) -> np.ndarray:
    """Window sums [BH, nW, d] of x [BH, N, d], each the exact sum rounded
    once to float64 (math.fsum).  For small problems."""
    import math

    bh, n, d = x.shape
    out = np.empty((bh, tok.shape[0], d))
    for b in range(bh):
        for w in range(tok.shape[0]):
            rows = x[b, tok[w][tok[w] >= 0]].astype(np.float64)
            for c in range(d):
                out[b, w, c] = math.fsum(rows[:, c].tolist())
    return out


def scores_in_channel_order(sq: np.ndarray, sk: np.ndarray) -> np.ndarray:
    """score[bh, i, j] = sum over channels c, in order, of sq[bh, i, c] *
    sk[bh, j, c], each product and each sum rounded to float64 on its own
    (numpy element-wise operations: no fused multiply-add)."""
    acc = np.zeros((sq.shape[0], sq.shape[1], sk.shape[1]))
    for c in range(sq.shape[2]):
        acc = acc + sq[:, :, None, c] * sk[:, None, :, c]
    return acc


def near_ties(scores: np.ndarray, topk: int, wgrid, radius: int = -1, rel: float = 1e-9) -> int:
    """Count of (head, window) rows whose ranking of candidates could change
    under float64 rounding: two candidates adjacent in score order, at
    positions r and r + 1 with r < topk (they decide the routed set or its
    listed order), whose scores differ by at most rel * the row's largest
    |score|.  scores [BH, nW, nW]; candidates as in route_topk."""
    bh, nw, _ = scores.shape
    if radius >= 0:
        pos = np.stack(np.unravel_index(np.arange(nw), tuple(wgrid)), axis=1)
        near = (np.abs(pos[:, None, :] - pos[None, :, :]) <= radius).all(axis=2)
    count = 0
    for b in range(bh):
        for i in range(nw):
            cand = [j for j in range(nw) if j != i and (radius < 0 or near[i, j])]
            s = np.sort(scores[b, i, cand])[::-1]
            tol = rel * max(np.abs(s).max(), 1e-300)
            gaps = s[:-1] - s[1:]
            if (gaps[:min(topk, len(gaps))] <= tol).any():
                count += 1
    return count
