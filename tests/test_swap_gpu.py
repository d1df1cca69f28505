"""GPU per-block random swap (het_attn_swap) against the oracle, bit-exact.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): at every transformer block some uncertain tokens trade
places with randomly chosen certain ones (§3.2.2, after Eq. 12), at the swap
ratio r of App. B (Random Token Percentage, Table 8; 7 % over 30 blocks).

Every route a launch writes (masks, index lists, counts) is compared with the
oracle's route for the same block; thresholds must be copied from the input.
The sizes cover every register layout of the kernel (N up to 8192, 16384,
32768, 65536, and the re-reading form above), ragged rows, several samples,
the in-place form, all 32-bit counter and key words, and two tokens with equal
draws at the selection boundary (golden/swap_ties.json).
"""
import ctypes

import numpy as np
import pytest

import uncertainty_routed_heterogeneous_amd as het
import workloads as W
from gpu_util import assert_close, assert_route_equal, gpu_forward, gpu_route, log, route_to_numpy, to_gpu
from swap_cases import random_mask, tie_cases, tie_mask

pytestmark = pytest.mark.gpu

SEED = 0x1234_5678_9ABC_DEF0


def route_from_mask(mask: np.ndarray, grid, dense_count_host=None, thresh=None):
    """A GPU route whose mask is `mask` (the swap reads nothing else but the
    thresholds)."""
    import torch
    B, N = mask.shape
    dev = torch.device("cuda")
    th = np.arange(B, dtype=np.float64) + 0.25 if thresh is None else thresh
    if dense_count_host is None:
        k = np.count_nonzero(mask == 0, axis=1)
        dense_count_host = int(k[0]) if np.all(k == k[0]) else -1
    return het.Route(to_gpu(mask.astype(np.uint8)),
                     torch.full((B, N), -7, dtype=torch.int32, device=dev),
                     torch.full((B, N), -7, dtype=torch.int32, device=dev),
                     torch.zeros((B, 2), dtype=torch.int32, device=dev),
                     to_gpu(np.ascontiguousarray(th, dtype=np.float64)), dense_count_host,
                     tuple(grid), (1, 1, 1))


def check_swap(oracle_mod, r_in, mask_in, ratio, seed, step, block, n_blocks, what=""):
    import torch
    log(f"[swap] {what} B={mask_in.shape[0]} N={mask_in.shape[1]} r={ratio} seed={seed:#x} "
        f"step={step} block={block} n_blocks={n_blocks}")
    thresh_in = r_in.thresh.cpu().numpy()
    outs = het.swap(r_in, ratio, seed, step, block, n_blocks)
    torch.cuda.synchronize()
    assert len(outs) == n_blocks
    for l, o in enumerate(outs):
        ref = oracle_mod.route_swap(mask_in, ratio, seed, step, (block + l) & 0xFFFFFFFF)
        g = route_to_numpy(o)
        assert_route_equal(g, ref, exact_thresh=False)
        np.testing.assert_array_equal(g["thresh"], thresh_in)
        assert o.dense_count_host == r_in.dense_count_host
        np.testing.assert_array_equal(g["counts"][:, 0], np.count_nonzero(mask_in == 0, axis=1))
    return outs


@pytest.mark.parametrize("name", ["tiny", "wan13b", "wan5b", "long"])
def test_swap_workloads(oracle_mod, name):
    """30 blocks at r = 7 % from the workload's top-rho route."""
    w = W.WORKLOADS[name]
    u = W.make_u(w)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=w.rho)
    mask = oracle_mod.route_top_rho(u, w.rho).mask
    np.testing.assert_array_equal(r.mask.cpu().numpy(), mask)
    outs = check_swap(oracle_mod, r, mask, 0.07, SEED, 3, 0, 30, name)
    # Different blocks move different tokens.
    if w.n_tokens > 1000:
        assert not np.array_equal(outs[0].mask.cpu().numpy(), outs[1].mask.cpu().numpy())


@pytest.mark.parametrize("ratio", [0.0, 0.5 / 32760, 1.0 / 32760, 0.07, 0.2, 0.5, 1.0])
def test_swap_ratios(oracle_mod, ratio):
    """r from none to all: S is capped by the smaller set (here the dense one)."""
    w = W.WORKLOADS["wan13b"]
    u = W.make_u(w)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=w.rho)
    mask = r.mask.cpu().numpy()
    outs = check_swap(oracle_mod, r, mask, ratio, SEED, 11, 7, 2, f"ratio {ratio}")
    moved = int(np.count_nonzero(outs[0].mask.cpu().numpy() != mask))
    S = min(int(np.floor(ratio * w.n_tokens + 0.5)), 6552, w.n_tokens - 6552)
    assert moved == 2 * S


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 1000, 8192, 8193, 16384, 16385, 32768, 32769,
                               65536, 65537, 200000])
def test_swap_sizes(oracle_mod, N):
    B = 2 if N <= 65537 else 1
    mask = random_mask(B, N, 0.3, seed=N, local_value=1 if N % 2 else 255)
    r = route_from_mask(mask, (1, 1, N))
    check_swap(oracle_mod, r, mask, 0.1, SEED ^ N, 1, 4, 3, f"N={N}")


@pytest.mark.parametrize("kind", ["all_dense", "all_local", "one_dense", "one_local"])
def test_swap_degenerate_masks(oracle_mod, kind):
    N = 4 * 8 * 8
    mask = np.ones((2, N), np.uint8) if kind in ("all_local", "one_dense") else np.zeros((2, N), np.uint8)
    if kind == "one_dense":
        mask[:, [17, 200]] = 0
        mask[1, 200] = 1
    if kind == "one_local":
        mask[:, [3, 255]] = 1
        mask[1, 3] = 0
    r = route_from_mask(mask, (4, 8, 8), dense_count_host=-1)
    for ratio in (0.07, 1.0):
        outs = check_swap(oracle_mod, r, mask, ratio, SEED, 0, 0, 2, kind)
        moved = np.count_nonzero(outs[0].mask.cpu().numpy() != mask, axis=1)
        nd = np.count_nonzero(mask == 0, axis=1)
        S = np.minimum(np.minimum(int(np.floor(ratio * N + 0.5)), nd), N - nd)
        np.testing.assert_array_equal(moved, 2 * S)
        assert (kind.startswith("all") and S.max() == 0) or S.min() >= 1


def test_swap_in_place(oracle_mod):
    import torch
    w = W.WORKLOADS["wan13b"]
    u = W.make_u(w)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, rho=w.rho)
    mask = r.mask.cpu().numpy()
    th = r.thresh.cpu().numpy()
    log("[swap] in place, wan13b")
    (o,) = het.swap(r, 0.07, SEED, 2, 9, in_place=True)
    torch.cuda.synchronize()
    assert o is r
    assert_route_equal(route_to_numpy(r), oracle_mod.route_swap(mask, 0.07, SEED, 2, 9),
                       exact_thresh=False)
    np.testing.assert_array_equal(r.thresh.cpu().numpy(), th)
    # The form that re-reads the mask (N > 65536), in place.
    N = 100003
    m2 = random_mask(1, N, 0.25, seed=5)
    r2 = route_from_mask(m2, (1, 1, N))
    log(f"[swap] in place, N={N}")
    het.swap(r2, 0.2, SEED, 0, 1, in_place=True)
    torch.cuda.synchronize()
    assert_route_equal(route_to_numpy(r2), oracle_mod.route_swap(m2, 0.2, SEED, 0, 1),
                       exact_thresh=False)


@pytest.mark.parametrize("seed,step,block", [(0, 0, 0), (0xFFFFFFFF, 1, 2), (1 << 32, 7, 0),
                                             ((1 << 64) - 1, 0xFFFFFFFF, 0xFFFFFFFE)])
def test_swap_counter_and_key_words(oracle_mod, seed, step, block):
    """Every word of the seed and counters, and block numbers wrapping at 2^32."""
    N = 3 * 30 * 52
    mask = random_mask(2, N, 0.2, seed=9)
    r = route_from_mask(mask, (3, 30, 52))
    check_swap(oracle_mod, r, mask, 0.07, seed, step, block, 3, "words")


@pytest.mark.parametrize("idx", range(4))
def test_swap_equal_draws(oracle_mod, idx):
    """Equal draws at the boundary: the lower token index moves first."""
    case = tie_cases()[idx]
    mask = tie_mask(oracle_mod, case)
    r = route_from_mask(mask, (1, 1, case["N"]))
    outs = check_swap(oracle_mod, r, mask, case["r"], case["seed"], case["step"], case["block"], 1,
                      f"tie {case['side']} N={case['N']}")
    m = outs[0].mask.cpu().numpy()[0]
    assert m[case["i"]] != mask[0, case["i"]] and m[case["j"]] == mask[0, case["j"]]


def test_swap_mean_std_route(oracle_mod):
    """Per-sample dense counts (mean-std threshold) stay per sample."""
    w = W.WORKLOADS["wan5b"]
    u = W.make_u(w)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, w.dtype, c=0.9)
    assert r.dense_count_host == -1
    mask = r.mask.cpu().numpy()
    check_swap(oracle_mod, r, mask, 0.07, SEED, 5, 0, 4, "mean-std wan5b")


def test_swap_null_thresholds(oracle_mod):
    """No output thresholds, or none to copy (NaN then)."""
    import torch
    N = 256
    mask = random_mask(1, N, 0.25, seed=1)
    r = route_from_mask(mask, (4, 8, 8))
    lib = het.load_library()
    shape = het.make_shape(1, 1, 64, (4, 8, 8), (1, 1, 1), het.HET_F32)
    out = [torch.empty((1, N), dtype=torch.uint8, device="cuda"),
           torch.empty((1, N), dtype=torch.int32, device="cuda"),
           torch.empty((1, N), dtype=torch.int32, device="cuda"),
           torch.empty((1, 2), dtype=torch.int32, device="cuda"),
           torch.zeros((1,), dtype=torch.float64, device="cuda")]
    ref = oracle_mod.route_swap(mask, 0.1, 3, 0, 0)
    log("[swap] null thresholds")
    for in_th, out_th in ((0, None), (None, 0)):
        rs_in = r.as_struct()
        if in_th is None:
            rs_in.thresh = None
        rs_out = het.RouteStruct(out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                                 out[3].data_ptr(), out[4].data_ptr() if out_th is not None else None, 0)
        st = lib.het_attn_swap(ctypes.byref(shape), ctypes.byref(rs_in), 0.1, 3, 0, 0, 1,
                               ctypes.byref(rs_out), None)
        assert st == het.HET_OK
        torch.cuda.synchronize()
        assert rs_out.dense_count_host == r.dense_count_host
        got = dict(mask=out[0].cpu().numpy(), dense_idx=out[1].cpu().numpy(),
                   local_idx=out[2].cpu().numpy(), counts=out[3].cpu().numpy())
        assert_route_equal(got, ref, exact_thresh=False)
    assert np.isnan(out[4].cpu().numpy()[0])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_swapped_route_forward(oracle_mod, dtype):
    """A swapped route drives the attention like any other route."""
    w = W.Workload("swapfwd", 950, 2, 2, 64, (4, 8, 12), (3, 5, 5), 0.3, dtype, "iid")
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, dtype, rho=w.rho)
    mask = r.mask.cpu().numpy()
    outs = check_swap(oracle_mod, r, mask, 0.1, SEED, 1, 0, 3, f"forward {dtype}")
    for o in outs:
        got = gpu_forward(q, k, v, o, dtype)
        ref = oracle_mod.forward(q, k, v, w.grid, w.window, w.softmax_scale, o.mask.cpu().numpy())
        assert_close(got, ref, dtype, f"swapped route {dtype}")
