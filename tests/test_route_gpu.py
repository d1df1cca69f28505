"""GPU route (threshold, mask, compaction) against the oracle, bit-exact.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT), §3.2.2 Eqs. 11-12."""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_route_equal, gpu_route, log, route_to_numpy

pytestmark = pytest.mark.gpu


def run_top_rho(oracle_mod, u, grid, rho, heads=2, head_dim=64, dtype="f32"):
    r = gpu_route(u, grid, (3, 3, 3), heads, head_dim, dtype, rho=rho)
    o = oracle_mod.route_top_rho(u, rho)
    g = route_to_numpy(r)
    assert_route_equal(g, o)
    assert r.dense_count_host == int(o.counts[0, 0])
    return g


@pytest.mark.parametrize("name", ["tiny", "wan13b", "wan5b", "long"])
def test_route_workloads(oracle_mod, name):
    w = W.WORKLOADS[name]
    u = W.make_u(w)
    log(f"[route] {name} B={w.batch} N={w.n_tokens} rho={w.rho}")
    g = run_top_rho(oracle_mod, u, w.grid, w.rho, w.heads, w.head_dim, w.dtype)
    assert np.all(g["counts"][:, 0] == W.dense_count(w.n_tokens, w.rho))


@pytest.mark.parametrize("rho", W.RHO_SWEEP)
def test_route_rho_sweep(oracle_mod, rho):
    w = W.WORKLOADS["wan13b"]
    log(f"[route] sweep rho={rho}")
    run_top_rho(oracle_mod, W.make_u(w), w.grid, rho, w.heads, w.head_dim, w.dtype)
    t = W.WORKLOADS["tiny"]
    run_top_rho(oracle_mod, W.make_u(t), t.grid, rho)


@pytest.mark.parametrize("kind", ["ties", "equal"])
@pytest.mark.parametrize("name", ["tiny", "wan13b"])
def test_route_ties(oracle_mod, kind, name):
    w = W.WORKLOADS[name]
    log(f"[route] {name} u={kind}")
    u = W.make_u(w, kind)
    g = run_top_rho(oracle_mod, u, w.grid, w.rho, w.heads, w.head_dim, w.dtype)
    if kind == "equal":
        k = W.dense_count(w.n_tokens, w.rho)
        assert g["dense_idx"][0, :k].tolist() == list(range(k))


@pytest.mark.parametrize("rho_n", ["zero", "one_token", "half", "all"])
def test_route_edge_rho(oracle_mod, rho_n):
    w = W.WORKLOADS["wan5b"]
    N = w.n_tokens
    rho = {"zero": 0.0, "one_token": 1.0 / N, "half": 0.5, "all": 1.0}[rho_n]
    log(f"[route] edge rho={rho}")
    run_top_rho(oracle_mod, W.make_u(w), w.grid, rho, w.heads, w.head_dim, w.dtype)


def test_route_special_values(oracle_mod):
    rng = np.random.default_rng(3)
    u = rng.random((2, 4 * 8 * 8)).astype(np.float32)
    u[0, [3, 77, 200]] = np.nan
    u[0, [5, 6, 150]] = np.inf
    u[1, ::7] = 0.0
    u[1, 1::7] = -0.0
    log("[route] NaN/inf/-0")
    for rho in (0.01, 0.25, 0.9):
        run_top_rho(oracle_mod, u, (4, 8, 8), rho)


def test_route_single_token_and_small(oracle_mod):
    log("[route] N=1, N=3")
    run_top_rho(oracle_mod, np.array([[0.3]], np.float32), (1, 1, 1), 1.0)
    run_top_rho(oracle_mod, np.array([[0.3]], np.float32), (1, 1, 1), 0.0)
    run_top_rho(oracle_mod, np.array([[0.3, 0.1, 0.3]], np.float32), (1, 1, 3), 0.5)


def test_route_mean_std_crafted(oracle_mod):
    u = np.tile(np.array([0.0, 2.0], np.float32), 128)[None, :]  # mu = 1, sigma = 1
    for c in (0.5, 1.0, -1.0, 3.0):
        log(f"[route] mean-std crafted c={c}")
        r = gpu_route(u, (4, 8, 8), (3, 3, 3), 2, 64, "f32", c=c)
        assert r.dense_count_host == -1
        assert_route_equal(route_to_numpy(r), oracle_mod.route_mean_std(u, c))


def check_mean_std(oracle_mod, u, grid, c, heads=2, head_dim=64, dtype="f32", window=(3, 3, 3)):
    """The GPU sums in a different (fixed) order than the oracle; a token may
    only differ if its u lies within rounding distance of T."""
    r = gpu_route(u, grid, window, heads, head_dim, dtype, c=c)
    g = route_to_numpy(r)
    o = oracle_mod.route_mean_std(u, c)
    np.testing.assert_allclose(g["thresh"], o.thresh, rtol=1e-13, atol=0)
    diff = g["mask"] != o.mask
    if diff.any():
        b, i = np.nonzero(diff)
        near = np.abs(u[b, i].astype(np.float64) - o.thresh[b]) <= 1e-12 * np.abs(o.thresh[b])
        assert near.all(), "mask differs away from the threshold"
        log(f"  {diff.sum()} tokens at the threshold differ by rounding")
    else:
        assert_route_equal(g, o, exact_thresh=False)


@pytest.mark.parametrize("name", ["tiny", "wan13b", "wan5b"])
def test_route_mean_std_workloads(oracle_mod, name):
    w = W.WORKLOADS[name]
    log(f"[route] mean-std {name} c=0.9")
    check_mean_std(oracle_mod, W.make_u(w), w.grid, 0.9, w.heads, w.head_dim, w.dtype, w.window)


@pytest.mark.parametrize("n", [8192, 8193, 16385, 32768, 32769, 65536, 65537, 100003])
def test_route_chunk_lengths(oracle_mod, n):
    """Sample lengths at the edges of the per-thread chunk lengths of the
    route kernel (keys held in registers up to 65536 tokens, re-read from
    memory beyond).  Sample 0 has both signs (keys differ in the top bit),
    sample 1 has 51 distinct values (long runs of ties)."""
    rng = np.random.default_rng(n)
    u = np.empty((2, n), np.float32)
    u[0] = rng.standard_normal(n)
    u[1] = np.round(rng.random(n) * 50) / 50
    for rho in (0.2, 0.73):
        log(f"[route] N={n} rho={rho}")
        run_top_rho(oracle_mod, u, (1, 1, n), rho)
    log(f"[route] N={n} mean-std c=0.5")
    check_mean_std(oracle_mod, u, (1, 1, n), 0.5)


def test_route_keys_one_ulp_apart(oracle_mod):
    """All keys share their top 31 bits: the select has a single 1-bit digit."""
    a = np.float32(1.0)
    b = np.nextafter(a, np.float32(2.0))
    rng = np.random.default_rng(5)
    u = np.where(rng.random((2, 1000)) < 0.5, a, b).astype(np.float32)
    for rho in (0.1, 0.5, 0.9):
        log(f"[route] one-ulp keys rho={rho}")
        run_top_rho(oracle_mod, u, (1, 1, 1000), rho)


def test_route_deterministic():
    w = W.WORKLOADS["long"]
    u = W.make_u(w, "ties")
    a = route_to_numpy(gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=0.2))
    b = route_to_numpy(gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=0.2))
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
