"""GPU heterogeneous attention against the fp64 oracle.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): Eq. 2 (dense), Eq. 3 (local), Eq. 13 (merge).

Tolerances (max-abs / mean-abs against the oracle): bf16 inputs 2e-2 / 2e-3,
fp32 inputs 1e-5 / 1e-6.  Small cases compare every output element; the
full-size workloads, run in the same launch configuration as the benchmark,
compare sampled dense and local rows that the oracle computes one by one.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_close, gpu_forward, gpu_route, log

pytestmark = pytest.mark.gpu


def small_case(grid, heads, head_dim, dtype, batch=2, seed=0, window=(3, 7, 7), rho=0.3,
               u_kind="iid"):
    w = W.Workload(f"case{seed}", 900 + seed, batch, heads, head_dim, tuple(grid), tuple(window),
                   rho, dtype, u_kind)
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    return w, q, k, v, u


def full_parity(oracle_mod, w, q, k, v, u, rho=None, c=None, what=""):
    log(f"[forward] {what} grid={w.grid} win={w.window} B={w.batch} H={w.heads} D={w.head_dim} "
        f"{w.dtype} rho={rho} c={c}")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=rho, c=c)
    got = gpu_forward(q, k, v, r, w.dtype, prefill=float("nan"))
    mask = r.mask.cpu().numpy()
    ref = oracle_mod.forward(q, k, v, w.grid, w.window, w.softmax_scale, mask)
    assert_close(got, ref, w.dtype, what)
    return got, ref, mask


def test_tiny_workload(oracle_mod):
    w = W.WORKLOADS["tiny"]
    q, k, v = W.make_qkv(w)
    full_parity(oracle_mod, w, q, k, v, W.make_u(w), rho=w.rho, what="tiny")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("rho", [0.0, 0.3, 1.0])
def test_small_grid_all_rows(oracle_mod, dtype, head_dim, rho):
    # N = 1200: several 128-query tiles with a ragged last one, and N % 64 != 0.
    w, q, k, v, u = small_case((6, 10, 20), 3, head_dim, dtype, seed=head_dim + int(10 * rho))
    full_parity(oracle_mod, w, q, k, v, u, rho=rho, what="small")


@pytest.mark.parametrize("window", [(1, 3, 3), (3, 5, 9), (5, 7, 11), (3, 9, 25)])
def test_window_shapes(oracle_mod, window):
    # Ragged grid in every axis; windows up to the widest the local kernel takes.
    w, q, k, v, u = small_case((5, 11, 27), 2, 64, "bf16", seed=7, window=window)
    full_parity(oracle_mod, w, q, k, v, u, rho=0.2, what=f"window {window}")


@pytest.mark.parametrize("grid", [(4, 9, 40), (4, 9, 14), (4, 9, 52)])
def test_local_workgroup_shapes_all_rows(oracle_mod, grid):
    """The local kernel's three workgroup shapes at the 3x7x7 window, each on
    every row of a ragged grid: 5 column tiles of 8 take one frame x 8 x-tiles
    in eight waves, 2 take two frames x 4 x-tiles, 7 take one frame x 4
    x-tiles in four-wave workgroups, two to a CU."""
    w, q, k, v, u = small_case(grid, 2, 128, "bf16", seed=300 + grid[2])
    full_parity(oracle_mod, w, q, k, v, u, rho=0.2, what=f"workgroup shape, grid {grid}")


@pytest.mark.parametrize("window", [(9, 9, 9), (11, 11, 11), (13, 13, 13)])
@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("f32", 64)])
def test_cubic_windows_all_rows(oracle_mod, window, dtype, head_dim):
    """The window ablation's neighbourhoods ([HetA] Table 7; 11^3 is the
    default): every row of a ragged grid larger than the window in each axis."""
    w, q, k, v, u = small_case((15, 18, 29), 2, head_dim, dtype, batch=1, seed=20 + window[0],
                               window=window)
    full_parity(oracle_mod, w, q, k, v, u, rho=0.2, what=f"window {window}")


def test_window_covering_grid_equals_dense(oracle_mod):
    w, q, k, v, u = small_case((3, 4, 5), 2, 128, "f32", batch=1, seed=8, window=(5, 9, 11))
    got_local, ref, _ = full_parity(oracle_mod, w, q, k, v, u, rho=0.0, what="cover-local")
    got_dense, _, _ = full_parity(oracle_mod, w, q, k, v, u, rho=1.0, what="cover-dense")
    assert_close(got_local, got_dense.astype(np.float64), "f32", "local vs dense")


def test_unit_window_returns_values(oracle_mod):
    w, q, k, v, u = small_case((4, 6, 10), 2, 64, "bf16", seed=9, window=(1, 1, 1))
    log("[forward] 1x1x1 window")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=0.0)
    got = gpu_forward(q, k, v, r, w.dtype)
    np.testing.assert_array_equal(got, v)


def test_unit_values_give_unit_output():
    w, q, k, v, u = small_case((6, 10, 20), 3, 128, "bf16", seed=10)
    v = np.ones_like(v)
    log("[forward] V = 1")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=0.3)
    got = gpu_forward(q, k, v, r, w.dtype)
    assert np.abs(got - 1.0).max() <= 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token(oracle_mod, dtype):
    w, q, k, v, u = small_case((1, 1, 1), 1, 64, dtype, batch=1, seed=11, window=(3, 3, 3))
    for rho in (0.0, 1.0):
        full_parity(oracle_mod, w, q, k, v, u, rho=rho, what="N=1")


@pytest.mark.parametrize("rho", [1.0 / 1200, 0.01, 0.11])
def test_few_dense_tokens(oracle_mod, rho):
    """Less dense work than persistent workgroups, and tiles split across
    workgroups (the dense kernel's split-and-merge path)."""
    w, q, k, v, u = small_case((6, 10, 20), 3, 128, "bf16", seed=15)
    full_parity(oracle_mod, w, q, k, v, u, rho=rho, what=f"few dense rho={rho:.4f}")


def test_mean_std_route_forward(oracle_mod):
    w, q, k, v, u = small_case((6, 10, 20), 2, 128, "bf16", seed=12, u_kind="lognormal")
    full_parity(oracle_mod, w, q, k, v, u, c=0.9, what="mean-std")


def test_clustered_blobs(oracle_mod):
    w, q, k, v, u = small_case((8, 12, 24), 2, 128, "bf16", seed=13, u_kind="blobs")
    full_parity(oracle_mod, w, q, k, v, u, rho=0.2, what="blobs")


def test_medium_all_rows_split_units(oracle_mod):
    """Every element at 8192 tokens x 12 heads: 84 dense units for 256
    persistent workgroups, so every unit is cut into pieces of 42 key tiles
    that visit their tiles in rotated order and are merged; the route runs
    on 4 workgroups per sample."""
    w = W.Workload("medium", 950, 1, 12, 128, (8, 32, 32), (3, 7, 7), 0.2, "bf16", "iid")
    q, k, v = W.make_qkv(w)
    log("[forward] medium 8x32x32, 12 heads, every row")
    full_parity(oracle_mod, w, q, k, v, W.make_u(w), rho=0.2, what="medium")


def sampled_rows(mask_b: np.ndarray, n_each: int, rng) -> np.ndarray:
    dense = np.nonzero(mask_b == 0)[0]
    local = np.nonzero(mask_b == 1)[0]
    pick = []
    for group in (dense, local):
        if group.size:
            k = min(n_each, group.size)
            pick.extend([group[0], group[-1]])
            pick.extend(rng.choice(group, size=k, replace=False).tolist())
    return np.unique(np.array(pick, dtype=np.int64))


@pytest.mark.parametrize("name,rho", [("wan13b", 0.2), ("wan5b", 0.2), ("long", 0.2),
                                      ("wan13b", 1.0), ("wan13b", 0.05), ("wan13b_w11", 0.2),
                                      ("wan5b_w11", 0.2), ("wan13b_w11", 0.0)])
def test_full_size_sampled_rows(oracle_mod, name, rho):
    w = W.WORKLOADS[name]
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    log(f"[forward] full size {name} rho={rho} N={w.n_tokens}")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=rho)
    # Output prefilled with NaN: every row must be written exactly once
    # (Eq. 13), so no NaN may survive.
    got = gpu_forward(q, k, v, r, w.dtype, prefill=float("nan"))
    assert np.isfinite(got).all(), "an output element was not written"
    mask = r.mask.cpu().numpy()
    rng = np.random.default_rng(42)
    rows = np.concatenate([b * w.n_tokens + sampled_rows(mask[b], 40, rng) for b in range(w.batch)])
    ref = oracle_mod.attend_rows(q, k, v, w.grid, w.window, w.softmax_scale, mask, rows)
    got_rows = got.reshape(w.batch * w.n_tokens, w.heads, w.head_dim)[rows]
    assert_close(got_rows, ref, w.dtype, f"{name} sampled {rows.size} rows")


def test_deterministic():
    w, q, k, v, u = small_case((6, 10, 20), 3, 128, "bf16", seed=14)
    log("[forward] determinism")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=0.3)
    a = gpu_forward(q, k, v, r, w.dtype)
    b = gpu_forward(q, k, v, r, w.dtype)
    np.testing.assert_array_equal(a, b)
