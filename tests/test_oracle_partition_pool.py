"""Pins of the oracle's window partition and pooling (CPU only).

Partition: the BASA summary (paperlayer.ai, A.1) forms windows by a cyclic
shift, a reshape and a permute; the brute force applies exactly that recipe to
an array of token indices.  Invariant: every token lands in exactly one window
slot per block.  Pooling (sec. 3.2, A.1, "about 1/16 of the visual K/V for
pooling factors of 4") is pinned by a reshape-mean, the global mean at
pool = grid and the identity at pool = 1.
"""
import numpy as np
import pytest

from oracle import brute
from oracle.oracle import BO_ENOTDIV, BO_ERANGE, BO_EINVAL, Params
from video_gen_amd.synth import WORKLOADS, random_problem, random_short_problem


def _params(w, shift):
    return Params(1, 1, w.head_dim, w.grid, w.window, shift, w.pool, w.topk)


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("odd", [False, True])
def test_partition_matches_roll_reshape_permute(oracle_lib, name, odd):
    w = WORKLOADS[name]
    shift = w.shift if odd else (0, 0, 0)
    p = _params(w, shift)
    win_id, slot, tok = oracle_lib.partition(p)
    ref = brute.partition_tok(w.grid, w.window, shift)
    np.testing.assert_array_equal(tok, ref)
    # bijection: tok lists every token once (-1 past a short window's slots),
    # and (win_id, slot) inverts it
    n = p.n_tokens
    flat = tok.reshape(-1)
    real = flat >= 0
    assert np.array_equal(np.sort(flat[real]), np.arange(n))
    ws = np.repeat(np.arange(p.n_windows), p.window_tokens)[real]
    ss = np.tile(np.arange(p.window_tokens), p.n_windows)[real]
    np.testing.assert_array_equal(win_id[flat[real]], ws)
    np.testing.assert_array_equal(slot[flat[real]], ss)
    # every window holds its real slots: M unless the window does not divide
    counts = np.bincount(win_id, minlength=p.n_windows)
    np.testing.assert_array_equal(counts, oracle_lib.window_real_tokens(p))
    if not p.padded:
        assert np.all(counts == p.window_tokens)


def test_partition_random_small(oracle_lib):
    rng = np.random.default_rng(11)
    for _ in range(60):
        grid, window, shift, _ = random_problem(rng)
        p = Params(1, 1, 8, grid, window, shift)
        win_id, slot, tok = oracle_lib.partition(p)
        np.testing.assert_array_equal(tok, brute.partition_tok(grid, window, shift))
        assert np.array_equal(np.sort(tok.reshape(-1)), np.arange(p.n_tokens))


def test_shift_by_window_multiple_is_relabelling(oracle_lib):
    """A shift that is a multiple of the window gives the same windows as token sets."""
    grid, window = (2, 12, 16), (1, 4, 8)
    _, _, tok0 = oracle_lib.partition(Params(1, 1, 8, grid, window, (0, 0, 0)))
    _, _, tok1 = oracle_lib.partition(Params(1, 1, 8, grid, window, (1, 8, 8)))
    sets0 = sorted(tuple(sorted(r)) for r in tok0.tolist())
    sets1 = sorted(tuple(sorted(r)) for r in tok1.tolist())
    assert sets0 == sets1
    # a shift that is not a window multiple changes the partition
    _, _, tok2 = oracle_lib.partition(Params(1, 1, 8, grid, window, (0, 2, 3)))
    assert sorted(tuple(sorted(r)) for r in tok2.tolist()) != sets0


def test_shift_moves_window_origin(oracle_lib):
    """Window 0, slot 0 sits at the original coordinate equal to the shift."""
    grid, window, shift = (3, 8, 12), (1, 4, 4), (2, 3, 5)
    _, _, tok = oracle_lib.partition(Params(1, 1, 8, grid, window, shift))
    t, y, x = shift
    assert tok[0, 0] == (t * grid[1] + y) * grid[2] + x
    # the last slot of the last window wraps to (shift - 1) on every axis
    t, y, x = [(s - 1) % g for s, g in zip(shift, grid)]
    assert tok[-1, -1] == (t * grid[1] + y) * grid[2] + x


def test_validation_codes(oracle_lib):
    ok = Params(1, 1, 8, (1, 8, 8), (1, 4, 4), (0, 1, 2), (1, 2, 2), 1)
    assert oracle_lib.check(ok) == 0
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 3, 4))) == 0      # short windows
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 9, 4))) == BO_ERANGE
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 4, 4), pool=(1, 3, 2))) == BO_ENOTDIV
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 4, 4), shift=(0, 8, 0))) == BO_ERANGE
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 4, 4), topk=4)) == BO_ERANGE
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 4, 4), topk=3)) == 0
    assert oracle_lib.check(Params(1, 1, 0, (1, 8, 8), (1, 4, 4))) == BO_EINVAL
    assert oracle_lib.check(Params(1, 1, 8, (1, 8, 8), (1, 4, 4), scale=-1.0)) == BO_EINVAL


def _x(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("grid,pool", [((1, 32, 32), (1, 4, 4)), ((3, 10, 12), (3, 5, 4)),
                                       ((4, 6, 8), (2, 3, 1)), ((1, 16, 16), (1, 8, 8))])
def test_pool_matches_reshape_mean(oracle_lib, grid, pool):
    n = int(np.prod(grid))
    x = _x((2, 3, n, 16), 5)
    p = Params(2, 3, 16, grid, grid, (0, 0, 0), pool)
    got = oracle_lib.pool(p, x)
    ref = brute.pool_mean(x, grid, pool)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_pool_whole_grid_is_global_mean(oracle_lib):
    grid = (2, 8, 12)
    x = _x((1, 2, 192, 8), 6)
    p = Params(1, 2, 8, grid, grid, (0, 0, 0), grid)
    got = oracle_lib.pool(p, x)
    assert got.shape == (1, 2, 1, 8)
    np.testing.assert_allclose(got[:, :, 0], x.astype(np.float64).mean(axis=2), atol=1e-12)


def test_pool_unit_cell_is_identity(oracle_lib):
    grid = (2, 4, 6)
    x = _x((1, 1, 48, 8), 7)
    got = oracle_lib.pool(Params(1, 1, 8, grid, grid, (0, 0, 0), (1, 1, 1)), x)
    np.testing.assert_array_equal(got, x.astype(np.float64))


def test_pool_factor_four_keeps_one_sixteenth(oracle_lib):
    """4x4 pooling keeps 1/16 of the visual tokens (paperlayer.ai, A.1)."""
    for name in ("tiny", "flux1k"):
        w = WORKLOADS[name]
        p = _params(w, (0, 0, 0))
        assert p.pooled_tokens * 16 == p.n_tokens
        assert oracle_lib.load().bo_pooled_tokens(p.c()) * 16 == p.n_tokens


def test_pool_counts_at_workloads():
    assert {n: _params(w, (0, 0, 0)).pooled_tokens for n, w in WORKLOADS.items()} == {
        "tiny": 64, "flux1k": 256, "flux2k": 256, "flux4k": 256, "wan": 546, "wan_t3": 8190,
        "wan_t3w10": 8190, "flux2k_text": 256}


def _short_problem(rng, max_tokens=600):
    return random_short_problem(rng, max_tokens)


def test_partition_short_windows_match_padded_reshape(oracle_lib):
    """A window that does not divide the grid: roll, pad every axis with
    'no token' up to a window multiple, reshape, permute, and drop the padding
    (NumPy); the oracle's table must list the same tokens in the same order,
    every token exactly once, and (win_id, slot) must invert it."""
    rng = np.random.default_rng(21)
    for _ in range(30):
        grid, window, shift, _ = _short_problem(rng)
        p = Params(1, 1, 8, grid, window, shift)
        win_id, slot, tok = oracle_lib.partition(p)
        ref = brute.partition_tok(grid, window, shift)
        np.testing.assert_array_equal(tok, ref)
        real = tok[tok >= 0]
        assert np.array_equal(np.sort(real), np.arange(p.n_tokens))
        mw = oracle_lib.window_real_tokens(p)
        np.testing.assert_array_equal((tok >= 0).sum(axis=1), mw)
        for w in range(p.n_windows):
            np.testing.assert_array_equal(win_id[tok[w, :mw[w]]], w)
            np.testing.assert_array_equal(slot[tok[w, :mw[w]]], np.arange(mw[w]))
        # window extents: full, except the last along an axis the window does
        # not divide, which keeps the rest of the grid
        ext = [[w if c < -(-g // w) - 1 else g - c * w for c in range(-(-g // w))]
               for g, w in zip(grid, window)]
        expect = np.array([a * b * c for a in ext[0] for b in ext[1] for c in ext[2]])
        np.testing.assert_array_equal(mw, expect)
