"""Pins of the oracle's ablation routers and of the cut window border.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT).  §5.1 Routing Strategy and Table 6 compare the
uncertainty router with random routing (a fresh random subset per block) and
fixed uniform routing (an even, fixed pattern over the token volume); the
local window of Eq. 3 is a 3D neighbourhood whose border handling the pages
leave open.

Pins: the lattice property of the uniform pattern (every prefix of L tokens
holds ceil(L*K/N) dense ones; exact multiples; gaps), brute-force order
statistics of the draws for the random router, the tie cases of the swap
fixtures, frequencies over many blocks; the cut window against a
distance-based characterisation, and the cut-border attention against a
brute-force N x N masked softmax built from that characterisation.
"""
import itertools
import math

import numpy as np
import pytest

from swap_cases import tie_cases


def rho_count(N, rho):
    return min(max(int(math.floor(rho * N + 0.5)), 0), N)


# ------------------------------------------------------------- uniform ----

@pytest.mark.parametrize("N", [1, 2, 7, 10, 64, 256, 1000, 1023, 32760])
@pytest.mark.parametrize("rho", [0.0, 0.05, 0.2, 1.0 / 3.0, 0.5, 0.93, 1.0])
def test_uniform_prefix_counts(oracle_mod, N, rho):
    """Dense tokens form a lattice from token 0: any prefix of length L holds
    exactly ceil(L*K/N) of them (so no two prefixes of equal length differ by
    more than one, and the pattern starts at the first token)."""
    r = oracle_mod.route_uniform(2, N, rho)
    K = rho_count(N, rho)
    assert np.all(r.counts == [K, N - K])
    dense = (r.mask[0] == 0).astype(np.int64)
    prefix = np.concatenate([[0], np.cumsum(dense)])
    L = np.arange(N + 1, dtype=np.int64)
    np.testing.assert_array_equal(prefix, -((-L * K) // N))
    np.testing.assert_array_equal(r.mask[0], r.mask[1])  # same for every sample
    if K:
        gaps = np.diff(r.dense_idx[0, :K])
        assert np.all((gaps == N // K) | (gaps == -(-N // K)))


def test_uniform_exact_multiples_and_extremes(oracle_mod):
    r = oracle_mod.route_uniform(1, 100, 0.25)
    assert r.dense_idx[0, :25].tolist() == list(range(0, 100, 4))
    assert np.all(oracle_mod.route_uniform(1, 50, 0.0).mask == 1)
    assert np.all(oracle_mod.route_uniform(1, 50, 1.0).mask == 0)
    # rho*N = 2.5 rounds half up to 3
    assert oracle_mod.route_uniform(1, 10, 0.25).counts[0, 0] == 3


# -------------------------------------------------------------- random ----

@pytest.mark.parametrize("N", [1, 5, 64, 300])
@pytest.mark.parametrize("rho", [0.0, 0.1, 0.25, 1.0])
def test_random_is_the_k_smallest_draws(oracle_mod, N, rho):
    B, seed, step, block = 2, 0xABCDEF0123, 4, 9
    r = oracle_mod.route_random(B, N, rho, seed, step, block)
    K = rho_count(N, rho)
    for b in range(B):
        x = oracle_mod.swap_draws(N, b, seed, step, block)
        order = sorted(range(N), key=lambda i: (int(x[i]), i))
        assert sorted(order[:K]) == r.dense_idx[b, :K].tolist()
        assert r.counts[b].tolist() == [K, N - K]


def test_random_equal_draws_lower_index_first(oracle_mod):
    """Two tokens with equal draws at the boundary (swap fixtures): K = c + 1
    takes the lower index only."""
    for case in tie_cases():
        r = oracle_mod.route_random(1, case["N"], (case["c"] + 1) / case["N"], case["seed"],
                                    case["step"], case["block"])
        assert r.mask[0, case["i"]] == 0 and r.mask[0, case["j"]] == 1


def test_random_keyed_and_uniform_over_blocks(oracle_mod):
    N, rho, blocks = 2000, 0.2, 200
    hits = np.zeros(N)
    first = None
    for blk in range(blocks):
        r = oracle_mod.route_random(1, N, rho, 77, 1, blk)
        m = r.mask[0] == 0
        hits += m
        if first is None:
            first = m
        elif blk == 1:
            assert not np.array_equal(first, m)
    again = oracle_mod.route_random(1, N, rho, 77, 1, 0)
    np.testing.assert_array_equal(again.mask[0] == 0, first)
    # every token is dense with probability K/N per block; frequencies are
    # binomial(blocks, 0.2): mean exact, spread within 10 % of its variance
    p = 0.2
    assert hits.sum() == blocks * 400
    var = hits.var()
    assert abs(var - blocks * p * (1 - p)) < 0.1 * blocks * p * (1 - p)
    assert hits.min() > 0


# ---------------------------------------------------------- cut window ----

def brute_cut_window(S, k, pos):
    """Positions within Chebyshev distance (k-1)/2 of pos inside [0, S)."""
    inside = [j for j in range(S) if abs(j - pos) <= (k - 1) // 2]
    return inside[0], len(inside)


@pytest.mark.parametrize("S", range(1, 14))
@pytest.mark.parametrize("k", [1, 3, 5, 7, 9, 11, 13, 25])
def test_cut_window_matches_distance_definition(oracle_mod, S, k):
    for pos in range(S):
        assert oracle_mod.window_axis(S, k, pos, "truncate") == brute_cut_window(S, k, pos)


def test_cut_window_interior_and_total(oracle_mod):
    """Away from the border the cut and the shifted windows coincide; the
    cut removes h(h+1)/2 positions at each end in total (S >= k)."""
    for S, k in ((20, 7), (52, 11), (30, 13)):
        h = (k - 1) // 2
        for pos in range(h, S - h):
            assert oracle_mod.window_axis(S, k, pos, "truncate") == oracle_mod.window_axis(S, k, pos)
        total = sum(oracle_mod.window_axis(S, k, p, "truncate")[1] for p in range(S))
        assert total == S * k - h * (h + 1)


def brute_allowed_cut(grid, window, mask_row):
    T, H, W = grid
    N = T * H * W
    coords = np.array(list(itertools.product(range(T), range(H), range(W))))
    half = (np.array(window) - 1) // 2
    allowed = np.zeros((N, N), bool)
    for n in range(N):
        if mask_row[n] == 0:
            allowed[n] = True
        else:
            allowed[n] = np.all(np.abs(coords - coords[n]) <= half, axis=1)
    return allowed


def brute_forward_cut(q, k, v, grid, window, scale, mask):
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D))
    for b in range(B):
        allowed = brute_allowed_cut(grid, window, mask[b])
        for h in range(H):
            s = scale * (q[b, :, h, :].astype(np.float64) @ k[b, :, h, :].astype(np.float64).T)
            s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ v[b, :, h, :].astype(np.float64)
    return out


@pytest.mark.parametrize("grid,window", [((2, 3, 4), (1, 3, 3)), ((4, 8, 8), (3, 3, 3)),
                                         ((3, 5, 6), (3, 5, 1)), ((4, 8, 8), (3, 7, 7)),
                                         ((5, 6, 7), (5, 5, 9))])
@pytest.mark.parametrize("density", [0.0, 0.3])
def test_cut_forward_matches_bruteforce(oracle_mod, grid, window, density):
    T, Hg, Wg = grid
    N = T * Hg * Wg
    rng = np.random.default_rng(N)
    q, k, v = (rng.standard_normal((2, N, 2, 16)).astype(np.float32) for _ in range(3))
    mask = (rng.random((2, N)) >= density).astype(np.uint8)
    got = oracle_mod.forward(q, k, v, grid, window, 0.3, mask, border="truncate")
    ref = brute_forward_cut(q, k, v, grid, window, 0.3, mask)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_cut_weights_support(oracle_mod):
    grid, window = (4, 8, 8), (3, 5, 5)
    N = 256
    rng = np.random.default_rng(3)
    q, k = (rng.standard_normal((1, N, 1, 8)).astype(np.float32) for _ in range(2))
    mask = np.ones((1, N), np.uint8)
    allowed = brute_allowed_cut(grid, window, mask[0])
    for row in (0, 9, 100, 255):
        w = oracle_mod.attention_weights(q, k, grid, window, 0.5, mask, row, 0, border="truncate")
        assert np.all(w[~allowed[row]] == 0.0) and np.all(w[allowed[row]] > 0.0)
        assert abs(w.sum() - 1.0) < 1e-14
    # the corner token sees 2 x 3 x 3 keys, an interior one 3 x 5 x 5
    assert np.count_nonzero(allowed[0]) == 18
    assert np.count_nonzero(allowed[(1 * 8 + 3) * 8 + 3]) == 75
