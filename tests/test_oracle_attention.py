"""Pins for the oracle's attention (dense Eq. 2, local Eq. 3, merge Eq. 13).

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT), §3.1.1 Eqs. 2-3 and §3.2.2 Eq. 13.

Pins: torch's scaled_dot_product_attention (a library routine) for all-dense
and for windows covering the grid; a brute-force N x N masked softmax built
from an independently characterised window; closed forms (1x1x1 window,
Q = 0, V = 1); softmax weight ratios.
"""
import itertools

import numpy as np
import pytest
import torch


def brute_axis_window(S, k, pos):
    """The window along one axis, characterised without the clamp formula:
    among all length-min(k,S) intervals inside [0, S) that contain pos, the one
    whose centre is nearest to pos."""
    L = min(k, S)
    best = None
    for s in range(0, S - L + 1):
        if s <= pos < s + L:
            dist = abs((s + (L - 1) / 2.0) - pos)
            if best is None or dist < best[0]:
                best = (dist, s)
    return best[1], L


def brute_allowed(grid, window, mask_row):
    """[N, N] boolean: which keys each query may attend to."""
    T, H, W = grid
    N = T * H * W
    allowed = np.zeros((N, N), bool)
    coords = list(itertools.product(range(T), range(H), range(W)))
    for n, (t, y, x) in enumerate(coords):
        if mask_row[n] == 0:
            allowed[n, :] = True
            continue
        (t0, lt), (y0, ly), (x0, lx) = (brute_axis_window(T, window[0], t),
                                        brute_axis_window(H, window[1], y),
                                        brute_axis_window(W, window[2], x))
        for j, (tt, yy, xx) in enumerate(coords):
            if t0 <= tt < t0 + lt and y0 <= yy < y0 + ly and x0 <= xx < x0 + lx:
                allowed[n, j] = True
    return allowed


def brute_forward(q, k, v, grid, window, scale, mask):
    """Masked softmax over the full N x N score matrix, per sample and head."""
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D))
    for b in range(B):
        allowed = brute_allowed(grid, window, mask[b])
        for h in range(H):
            s = scale * (q[b, :, h, :].astype(np.float64) @ k[b, :, h, :].astype(np.float64).T)
            s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ v[b, :, h, :].astype(np.float64)
    return out


def sdpa(q, k, v, scale):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def rand_qkv(B, N, H, D, seed):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, N, H, D)).astype(np.float32) for _ in range(3))


@pytest.mark.parametrize("S", range(1, 13))
@pytest.mark.parametrize("k", [1, 3, 5, 7, 9, 11, 13, 15])
def test_window_axis_matches_bruteforce(oracle_mod, S, k):
    for pos in range(S):
        assert oracle_mod.window_axis(S, k, pos) == brute_axis_window(S, k, pos)


def test_window_axis_rejects_even_and_out_of_range(oracle_mod):
    for args in ((8, 4, 0), (8, 3, 8), (8, 3, -1), (0, 3, 0), (8, 0, 0)):
        with pytest.raises(ValueError):
            oracle_mod.window_axis(*args)


@pytest.mark.parametrize("grid,window", [((2, 3, 4), (1, 3, 3)), ((3, 3, 3), (3, 3, 3)),
                                         ((4, 8, 8), (3, 3, 3)), ((3, 5, 6), (3, 5, 1)),
                                         ((4, 8, 8), (3, 7, 7))])
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
def test_forward_matches_bruteforce_masked_softmax(oracle_mod, grid, window, density):
    T, Hg, Wg = grid
    N = T * Hg * Wg
    B, H, D = 2, 2, 16
    q, k, v = rand_qkv(B, N, H, D, seed=N + int(10 * density))
    rng = np.random.default_rng(7)
    mask = (rng.random((B, N)) >= density).astype(np.uint8)   # 1 = local
    scale = 0.3
    got = oracle_mod.forward(q, k, v, grid, window, scale, mask)
    ref = brute_forward(q, k, v, grid, window, scale, mask)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_all_dense_equals_library_sdpa(oracle_mod):
    """rho = 1: every token takes Eq. 2 over all keys = standard attention."""
    B, H, D, grid = 2, 3, 32, (3, 4, 5)
    N = 60
    q, k, v = rand_qkv(B, N, H, D, seed=11)
    mask = np.zeros((B, N), np.uint8)
    got = oracle_mod.forward(q, k, v, grid, (3, 3, 3), 1 / np.sqrt(D), mask)
    np.testing.assert_allclose(got, sdpa(q, k, v, 1 / np.sqrt(D)), rtol=1e-11, atol=1e-12)


def test_window_covering_grid_equals_library_sdpa(oracle_mod):
    """A window at least as large as the grid makes local = dense attention."""
    B, H, D, grid = 1, 2, 16, (3, 4, 5)
    N = 60
    q, k, v = rand_qkv(B, N, H, D, seed=12)
    mask = np.ones((B, N), np.uint8)
    for window in ((3, 5, 5), (5, 9, 11)):
        got = oracle_mod.forward(q, k, v, grid, window, 0.25, mask)
        np.testing.assert_allclose(got, sdpa(q, k, v, 0.25), rtol=1e-11, atol=1e-12)


def test_unit_window_returns_own_value(oracle_mod):
    B, H, D, grid = 1, 2, 8, (3, 4, 5)
    q, k, v = rand_qkv(B, 60, H, D, seed=13)
    mask = np.ones((B, 60), np.uint8)
    got = oracle_mod.forward(q, k, v, grid, (1, 1, 1), 0.5, mask)
    np.testing.assert_array_equal(got, v.astype(np.float64))


def test_zero_query_gives_window_mean(oracle_mod):
    """q = 0 makes every score equal, so o_i = mean of v over the key set."""
    B, H, D, grid, window = 1, 1, 4, (4, 6, 7), (3, 3, 5)
    T, Hg, Wg = grid
    N = T * Hg * Wg
    _, k, v = rand_qkv(B, N, H, D, seed=14)
    q = np.zeros_like(k)
    rng = np.random.default_rng(3)
    mask = (rng.random((B, N)) < 0.7).astype(np.uint8)
    got = oracle_mod.forward(q, k, v, grid, window, 1.0, mask)
    allowed = brute_allowed(grid, window, mask[0])
    for n in range(N):
        ref = v[0, allowed[n], 0, :].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(got[0, n, 0], ref, rtol=1e-13, atol=1e-14)


def test_unit_values_give_unit_output(oracle_mod):
    """v = 1: the weights of each row sum to one, so o = 1."""
    B, H, D, grid = 1, 2, 8, (4, 8, 8)
    q, k, _ = rand_qkv(B, 256, H, D, seed=15)
    v = np.ones_like(q)
    mask = (np.random.default_rng(1).random((B, 256)) < 0.75).astype(np.uint8)
    got = oracle_mod.forward(q, k, v, grid, (3, 3, 3), 0.125, mask)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)


def test_weights_support_sum_and_ratio(oracle_mod):
    B, H, D, grid, window = 1, 2, 16, (4, 8, 8), (3, 3, 3)
    N = 256
    q, k, _ = rand_qkv(B, N, H, D, seed=16)
    mask = (np.random.default_rng(2).random((B, N)) < 0.75).astype(np.uint8)
    allowed = brute_allowed(grid, window, mask[0])
    scale = 0.125
    for row in (0, 17, 100, 255):
        for head in range(H):
            w = oracle_mod.attention_weights(q, k, grid, window, scale, mask, row, head)
            assert np.all(w[~allowed[row]] == 0.0)
            assert np.all(w[allowed[row]] > 0.0)
            assert abs(w.sum() - 1.0) < 1e-14
            keys = np.nonzero(allowed[row])[0]
            s = scale * (k[0, keys, head, :].astype(np.float64) @ q[0, row, head, :].astype(np.float64))
            # softmax: w_j / w_0 = exp(s_j - s_0)
            np.testing.assert_allclose(w[keys] / w[keys[0]], np.exp(s - s[0]), rtol=1e-12)
            expect_m = 27 if mask[0, row] else N
            assert len(keys) == expect_m


def test_merge_selects_dense_or_local_rows(oracle_mod):
    """Eq. 13 with m in {0, 1}: each row equals the all-dense or all-local
    result for that row."""
    B, H, D, grid, window = 2, 2, 16, (4, 8, 8), (3, 3, 3)
    N = 256
    q, k, v = rand_qkv(B, N, H, D, seed=17)
    mask = (np.random.default_rng(4).random((B, N)) < 0.75).astype(np.uint8)
    got = oracle_mod.forward(q, k, v, grid, window, 0.125, mask)
    dense = oracle_mod.forward(q, k, v, grid, window, 0.125, np.zeros_like(mask))
    local = oracle_mod.forward(q, k, v, grid, window, 0.125, np.ones_like(mask))
    sel = mask[:, :, None, None].astype(bool)
    np.testing.assert_array_equal(got, np.where(sel, local, dense))


def test_attend_rows_subset_matches_forward(oracle_mod):
    B, H, D, grid = 2, 2, 16, (4, 8, 8)
    q, k, v = rand_qkv(B, 256, H, D, seed=18)
    mask = (np.random.default_rng(5).random((B, 256)) < 0.75).astype(np.uint8)
    full = oracle_mod.forward(q, k, v, grid, (3, 3, 3), 0.125, mask).reshape(B * 256, H, D)
    rows = np.array([0, 5, 255, 256, 400, 511])
    got = oracle_mod.attend_rows(q, k, v, grid, (3, 3, 3), 0.125, mask, rows)
    np.testing.assert_array_equal(got, full[rows])


def brute_row_lse(q, k, grid, window, scale, mask):
    """log sum_j exp(s_j) over the allowed keys of every row, [B, N, heads]."""
    B, N, H, D = q.shape
    out = np.zeros((B, N, H))
    for b in range(B):
        allowed = brute_allowed(grid, window, mask[b])
        for h in range(H):
            s = scale * (q[b, :, h, :].astype(np.float64) @ k[b, :, h, :].astype(np.float64).T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            out[b, :, h] = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


@pytest.mark.parametrize("grid,window", [((2, 3, 4), (1, 3, 3)), ((4, 8, 8), (3, 7, 7)), ((3, 5, 6), (3, 5, 1))])
def test_row_lse_matches_bruteforce(oracle_mod, grid, window):
    """The log of each row's softmax normaliser over an independently built key mask."""
    T, Hg, Wg = grid
    N = T * Hg * Wg
    B, H, D = 2, 2, 16
    q, k, _ = rand_qkv(B, N, H, D, seed=40 + N)
    mask = (np.random.default_rng(41).random((B, N)) >= 0.3).astype(np.uint8)
    rows = np.arange(B * N)
    got = oracle_mod.row_lse(q, k, grid, window, 0.3, mask, rows).reshape(B, N, H)
    np.testing.assert_allclose(got, brute_row_lse(q, k, grid, window, 0.3, mask), rtol=1e-12, atol=1e-12)


def test_row_lse_all_dense_equals_library_logsumexp(oracle_mod):
    B, H, D, grid = 1, 3, 32, (3, 4, 5)
    N = 60
    q, k, _ = rand_qkv(B, N, H, D, seed=42)
    mask = np.zeros((B, N), np.uint8)
    got = oracle_mod.row_lse(q, k, grid, (3, 3, 3), 0.2, mask, np.arange(N)).reshape(N, H)
    s = 0.2 * torch.einsum("nhd,mhd->hnm", torch.from_numpy(q[0]).double(), torch.from_numpy(k[0]).double())
    np.testing.assert_allclose(got, torch.logsumexp(s, dim=2).T.numpy(), rtol=1e-12, atol=1e-12)


def test_row_lse_closed_forms(oracle_mod):
    """Q = 0: every score is 0, so the LSE is the log of the key count (N for
    a dense row, the window's size for a local one); a 1x1x1 window: the
    query's score against its own key."""
    B, H, D, grid = 1, 2, 8, (4, 8, 8)
    N = 256
    q, k, _ = rand_qkv(B, N, H, D, seed=43)
    mask = np.ones((B, N), np.uint8)
    mask[0, ::5] = 0
    got = oracle_mod.row_lse(np.zeros_like(q), k, grid, (3, 5, 7), 0.7, mask, np.arange(N))
    want = np.where(mask[0] == 0, np.log(N), np.log(3 * 5 * 7))
    np.testing.assert_allclose(got, np.repeat(want[:, None], H, axis=1), rtol=1e-13)
    own = oracle_mod.row_lse(q, k, grid, (1, 1, 1), 0.7, np.ones((B, N), np.uint8), np.arange(N))
    np.testing.assert_allclose(own, 0.7 * np.einsum("nhd,nhd->nh", q[0].astype(np.float64), k[0].astype(np.float64)),
                               rtol=1e-12, atol=1e-12)
