"""GPU ablation routers and the cut window border against the oracle.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): the routing ablation of §5.1 (Routing Strategy,
Table 6) -- random routing per block and fixed uniform routing -- and the
border of the Eq. 3 neighbourhood, cut at the grid instead of shifted.

Routes are compared bit-exactly (mask, index lists, counts; thresholds are
NaN).  Outputs use the tolerances of the forward tests: bf16 2e-2 / 2e-3,
fp32 1e-5 / 1e-6 (max-abs / mean-abs against the fp64 oracle).
"""
import math

import numpy as np
import pytest

import uncertainty_routed_heterogeneous_amd as het
import workloads as W
from gpu_util import assert_close, assert_route_equal, gpu_forward, gpu_route, log, route_to_numpy
from swap_cases import tie_cases

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 256, 1000, 8192, 8193, 16385, 32760, 65536, 65537, 100003]


def check_nan_thresh(g):
    assert np.all(np.isnan(g["thresh"]))


@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("rho", [0.0, 0.05, 0.2, 1.0 / 3.0, 1.0])
def test_uniform_route(oracle_mod, N, rho):
    import torch
    log(f"[variants] uniform N={N} rho={rho:.4f}")
    r = het.route_uniform(2, (1, 1, N), (1, 1, 1), rho)
    torch.cuda.synchronize()
    g = route_to_numpy(r)
    ref = oracle_mod.route_uniform(2, N, rho)
    assert_route_equal(g, ref, exact_thresh=False)
    check_nan_thresh(g)
    assert r.dense_count_host == int(ref.counts[0, 0])


@pytest.mark.parametrize("N", SIZES)
def test_random_route(oracle_mod, N):
    import torch
    B = 2 if N <= 65536 else 1
    for rho, seed, step, block in ((0.2, 0x9E3779B97F4A7C15, 3, 0), (0.05, 1, 0, 29), (1.0, 7, 2, 5),
                                   (0.0, 7, 2, 5)):
        log(f"[variants] random N={N} rho={rho} seed={seed:#x} step={step} block={block}")
        outs = het.route_random(B, (1, 1, N), (1, 1, 1), rho, seed, step, block, n_blocks=3)
        torch.cuda.synchronize()
        for l, o in enumerate(outs):
            g = route_to_numpy(o)
            ref = oracle_mod.route_random(B, N, rho, seed, step, block + l)
            assert_route_equal(g, ref, exact_thresh=False)
            check_nan_thresh(g)
            assert o.dense_count_host == int(ref.counts[0, 0])


@pytest.mark.parametrize("idx", range(4))
def test_random_route_equal_draws(oracle_mod, idx):
    import torch
    case = tie_cases()[idx]
    N = case["N"]
    log(f"[variants] random tie case N={N}")
    (o,) = het.route_random(1, (1, 1, N), (1, 1, 1), (case["c"] + 1) / N, case["seed"], case["step"],
                            case["block"])
    torch.cuda.synchronize()
    m = o.mask.cpu().numpy()
    assert m[0, case["i"]] == 0 and m[0, case["j"]] == 1
    ref = oracle_mod.route_random(1, N, (case["c"] + 1) / N, case["seed"], case["step"], case["block"])
    np.testing.assert_array_equal(m, ref.mask)


def small_case(grid, heads, head_dim, dtype, batch=2, seed=0, window=(3, 7, 7), u_kind="iid"):
    w = W.Workload(f"var{seed}", 960 + seed, batch, heads, head_dim, tuple(grid), tuple(window),
                   0.3, dtype, u_kind)
    q, k, v = W.make_qkv(w)
    return w, q, k, v, W.make_u(w)


def cut_parity(oracle_mod, w, q, k, v, u, rho, what):
    log(f"[variants] cut border {what} grid={w.grid} win={w.window} {w.dtype} D={w.head_dim} rho={rho}")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=rho)
    import torch
    qg, kg, vg = (torch.from_numpy(x).to(torch.bfloat16 if w.dtype == "bf16" else torch.float32).cuda()
                  for x in (q, k, v))
    got = het.forward(qg, kg, vg, r, border="cut").float().cpu().numpy()
    mask = r.mask.cpu().numpy()
    ref = oracle_mod.forward(q, k, v, w.grid, w.window, w.softmax_scale, mask, border="truncate")
    assert_close(got, ref, w.dtype, what)
    return got, ref, mask


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
@pytest.mark.parametrize("window", [(3, 7, 7), (1, 3, 3), (5, 9, 13)])
def test_cut_border_all_rows(oracle_mod, dtype, head_dim, window):
    w, q, k, v, u = small_case((6, 10, 20), 2, head_dim, dtype, seed=head_dim + window[2], window=window)
    cut_parity(oracle_mod, w, q, k, v, u, 0.2, f"cut {window}")


@pytest.mark.parametrize("window", [(3, 9, 25), (5, 7, 11), (11, 11, 11), (13, 13, 13)])
def test_cut_border_wide_windows(oracle_mod, window):
    """Both tile shapes and both slot widths of the local kernel."""
    w, q, k, v, u = small_case((15, 18, 29), 1, 128, "bf16", batch=1, seed=40 + window[2],
                               window=window)
    cut_parity(oracle_mod, w, q, k, v, u, 0.2, f"cut {window}")


def test_cut_differs_from_shift_only_near_the_border(oracle_mod):
    """Interior tokens give the same output under both readings; tokens at
    the border differ (the pins of the two oracle readings, seen on the GPU)."""
    import torch
    w, q, k, v, u = small_case((6, 10, 20), 2, 64, "f32", seed=3, window=(3, 5, 5))
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=0.0)
    qg, kg, vg = (torch.from_numpy(x).cuda() for x in (q, k, v))
    a = het.forward(qg, kg, vg, r, border="cut").cpu().numpy().reshape(2, 6, 10, 20, 2, 64)
    b = het.forward(qg, kg, vg, r, border="shift").cpu().numpy().reshape(2, 6, 10, 20, 2, 64)
    np.testing.assert_allclose(a[:, 1:5, 2:8, 2:18], b[:, 1:5, 2:8, 2:18], rtol=0, atol=1e-6)
    assert np.abs(a[:, 0, 0, 0] - b[:, 0, 0, 0]).max() > 1e-3


@pytest.mark.parametrize("name", ["wan13b", "wan13b_w11"])
def test_cut_border_full_size_sampled(oracle_mod, name):
    w = W.WORKLOADS[name]
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    log(f"[variants] cut border full size {name}")
    import torch
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=w.rho)
    qg, kg, vg = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    got = het.forward(qg, kg, vg, r, border="cut").float().cpu().numpy()
    mask = r.mask.cpu().numpy()
    T, H, Wd = w.grid
    # border tokens (corners, edges, first and last frames) plus random ones
    rng = np.random.default_rng(5)
    idx = [0, Wd - 1, (H - 1) * Wd, H * Wd - 1, (T - 1) * H * Wd, T * H * Wd - 1,
           (T // 2 * H + 1) * Wd + 2]
    idx += rng.choice(w.n_tokens, size=60, replace=False).tolist()
    rows = np.unique(np.array(idx, dtype=np.int64))
    ref = oracle_mod.attend_rows(q, k, v, w.grid, w.window, w.softmax_scale, mask, rows, border="truncate")
    got_rows = got.reshape(w.n_tokens, w.heads, w.head_dim)[rows]
    assert_close(got_rows, ref, w.dtype, f"{name} cut border, {rows.size} rows")


@pytest.mark.parametrize("router", ["uniform", "random"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_on_ablation_routes(oracle_mod, router, dtype):
    import torch
    w, q, k, v, u = small_case((6, 10, 20), 2, 128, dtype, seed=11)
    if router == "uniform":
        r = het.route_uniform(2, w.grid, w.window, 0.2)
    else:
        (r,) = het.route_random(2, w.grid, w.window, 0.2, 99, 1, 4)
    torch.cuda.synchronize()
    log(f"[variants] forward on {router} route, {dtype}")
    got = gpu_forward(q, k, v, r, dtype)
    ref = oracle_mod.forward(q, k, v, w.grid, w.window, w.softmax_scale, r.mask.cpu().numpy())
    assert_close(got, ref, dtype, f"{router} route")
    assert r.dense_count_host == math.floor(0.2 * 1200 + 0.5)
