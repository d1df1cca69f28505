"""Pins for the oracle's routing (threshold, mask, compaction).

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT).  Routing rule: §3.2.2 Eqs. 11-12; dense fraction rho:
§3.2.2, text of Eq. 14.

Each pin is independent of the oracle's code: a brute-force Python ``sorted``,
closed forms on crafted inputs, and a normal-distribution tail probability.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def brute_top_rho(u_row, rho):
    """Dense set by plain Python: sort (-u, i), take the first round-half-up(rho*N)."""
    n = len(u_row)
    k = int(math.floor(rho * n + 0.5))
    k = max(0, min(n, k))

    def key(i):
        x = float(u_row[i])
        if math.isnan(x):
            x = math.inf
        return (-x, i)

    order = sorted(range(n), key=key)
    dense = set(order[:k])
    t = math.inf if k == 0 else -key(order[k - 1])[0]
    return dense, t


def check_route_consistency(r, B, N):
    for b in range(B):
        nd, nl = r.counts[b]
        assert nd + nl == N
        di = r.dense_idx[b, :nd]
        li = r.local_idx[b, :nl]
        assert np.all(np.diff(di) > 0) and np.all(np.diff(li) > 0)
        assert np.all(r.dense_idx[b, nd:] == -1) and np.all(r.local_idx[b, nl:] == -1)
        assert np.array_equal(np.sort(np.concatenate([di, li])), np.arange(N))
        assert np.all(r.mask[b, di] == 0) and np.all(r.mask[b, li] == 1)


@pytest.mark.parametrize("N", [1, 2, 7, 64, 256, 1000])
@pytest.mark.parametrize("rho", [0.0, 0.05, 0.1, 0.2, 0.25, 0.4, 0.5, 1.0])
def test_top_rho_matches_bruteforce(oracle_mod, N, rho):
    rng = np.random.default_rng(N * 100 + int(rho * 100))
    B = 3
    u = rng.random((B, N)).astype(np.float32)
    u[1] = np.floor(u[1] * 8) / 8  # many ties in sample 1
    r = oracle_mod.route_top_rho(u, rho)
    check_route_consistency(r, B, N)
    for b in range(B):
        dense, t = brute_top_rho(u[b], rho)
        assert set(r.dense_idx[b, : r.counts[b, 0]].tolist()) == dense
        assert r.thresh[b] == t


def test_top_rho_tiny_sweep_counts(oracle_mod):
    # round half up of rho*N at N = 256 (rho*N = 12.8, 25.6, 51.2, 102.4, 256)
    u = np.random.default_rng(0).random((1, 256)).astype(np.float32)
    got = [int(oracle_mod.route_top_rho(u, rho).counts[0, 0]) for rho in (0.05, 0.1, 0.2, 0.4, 1.0)]
    assert got == [13, 26, 51, 102, 256]


def test_top_rho_equal_u_takes_lowest_indices(oracle_mod):
    u = np.full((2, 100), 0.37, np.float32)
    r = oracle_mod.route_top_rho(u, 0.3)
    for b in range(2):
        assert r.dense_idx[b, :30].tolist() == list(range(30))
        assert r.thresh[b] == np.float32(0.37)


def test_top_rho_increasing_u_takes_last(oracle_mod):
    u = np.arange(50, dtype=np.float32)[None, :] / 50
    r = oracle_mod.route_top_rho(u, 0.2)
    assert r.dense_idx[0, :10].tolist() == list(range(40, 50))


def test_top_rho_special_values(oracle_mod):
    # NaN ranks as +inf (most uncertain); -0 equals +0 and ties fall to the index.
    u = np.array([[0.5, np.nan, -0.0, 0.0, np.inf, 0.25, 0.0, 1.0]], np.float32)
    r = oracle_mod.route_top_rho(u, 3 / 8)
    assert r.dense_idx[0, :3].tolist() == [1, 4, 7]
    assert r.thresh[0] == 1.0
    r = oracle_mod.route_top_rho(u, 7 / 8)
    # zeros at indices 2, 3, 6: the first two (by index) go dense
    assert r.dense_idx[0, :7].tolist() == [0, 1, 2, 3, 4, 5, 7]
    assert r.thresh[0] == 0.0


def test_top_rho_rejects_bad_rho(oracle_mod):
    u = np.zeros((1, 4), np.float32)
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle_mod.route_top_rho(u, bad)


def test_mean_std_closed_form(oracle_mod):
    # Half 0s and half 2s: mu = 1 and sigma = 1 exactly, so T = 1 + c.
    u = np.tile(np.array([0.0, 2.0], np.float32), 50)[None, :]
    r = oracle_mod.route_mean_std(u, 0.5)            # T = 1.5: the 2s are dense
    assert r.thresh[0] == 1.5
    assert r.dense_idx[0, : r.counts[0, 0]].tolist() == list(range(1, 100, 2))
    r = oracle_mod.route_mean_std(u, 1.0)            # T = 2: u = T is not < T -> dense
    assert r.counts[0, 0] == 50
    r = oracle_mod.route_mean_std(u, 1.0000001)      # T just above 2: nothing dense
    assert r.counts[0, 0] == 0
    r = oracle_mod.route_mean_std(u, -1.0)           # T = 0: every token dense
    assert r.counts[0, 0] == 100
    check_route_consistency(r, 1, 100)


def test_mean_std_gaussian_tail_matches_page_operating_point(oracle_mod):
    """For i.i.d. normal u the dense fraction is 1 - Phi(c).  At the page's
    c = 0.9 this is 18.4%, i.e. about 80% local (§5.1)."""
    with open(GOLDEN) as f:
        g = json.load(f)
    c = g["c_operating_point"]["c"]
    N = 400_000
    u = (np.random.default_rng(5).standard_normal((1, N)) + 10.0).astype(np.float32)
    r = oracle_mod.route_mean_std(u, c)
    frac = r.counts[0, 0] / N
    expect = 0.5 * math.erfc(c / math.sqrt(2.0))
    se = math.sqrt(expect * (1 - expect) / N)
    assert abs(frac - expect) < 6 * se + 1e-4
    assert abs((1 - frac) - g["c_operating_point"]["local_fraction_approx"]) < 0.03
    check_route_consistency(r, 1, N)


def test_page_local_only_router(oracle_mod):
    """The routing study's local-only row (§5.1, Routing Strategy, Table 6):
    rho = 0 routes no token to dense attention, so the layer is pure local
    attention (Eq. 13 with m = 1 everywhere)."""
    with open(GOLDEN) as f:
        rho = json.load(f)["local_only_router"]["rho"]
    grid, window, N = (3, 4, 5), (3, 3, 3), 60
    u = np.random.default_rng(21).random((2, N)).astype(np.float32)
    r = oracle_mod.route_top_rho(u, rho)
    assert (r.counts[:, 0] == 0).all() and (r.mask == 1).all() and (r.dense_idx == -1).all()
    rng = np.random.default_rng(22)
    q, k, v = (rng.standard_normal((2, N, 2, 8)).astype(np.float32) for _ in range(3))
    got = oracle_mod.forward(q, k, v, grid, window, 0.3, r.mask)
    local = oracle_mod.forward(q, k, v, grid, window, 0.3, np.ones((2, N), np.uint8))
    np.testing.assert_array_equal(got, local)


def test_mean_std_rejects_nonfinite_c(oracle_mod):
    u = np.zeros((1, 4), np.float32)
    for bad in (float("nan"), float("inf")):
        with pytest.raises(ValueError):
            oracle_mod.route_mean_std(u, bad)


def test_page_dense_fraction_counts(oracle_mod):
    """rho = 0.2 (§3.2.2 text of Eq. 14) on the two model grids gives exact
    integer dense counts."""
    with open(GOLDEN) as f:
        rho = json.load(f)["dense_fraction_approx"]["value"]
    for n, expect in ((21 * 30 * 52, 6552), (31 * 22 * 40, 5456), (41 * 30 * 52, 12792)):
        u = np.random.default_rng(n).random((1, n)).astype(np.float32)
        assert oracle_mod.route_top_rho(u, rho).counts[0, 0] == expect
