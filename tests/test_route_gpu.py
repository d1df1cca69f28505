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


# ---- top-rho over several workgroups per sample (N >= 8192): the workgroups
# exchange histograms and counts through the caller's workspace.

def route_via_abi(u_gpu, grid, rho, ws):
    """het_attn_route through the C ABI with a given workspace tensor."""
    import ctypes
    import torch
    import uncertainty_routed_heterogeneous_amd as het
    B, N = u_gpu.shape
    dev = u_gpu.device
    bufs = (torch.empty((B, N), dtype=torch.uint8, device=dev), torch.empty((B, N), dtype=torch.int32, device=dev),
            torch.empty((B, N), dtype=torch.int32, device=dev), torch.empty((B, 2), dtype=torch.int32, device=dev),
            torch.empty((B,), dtype=torch.float64, device=dev))
    rs = het.RouteStruct(*(b.data_ptr() for b in bufs), -1)
    shape = het.make_shape(B, 2, 64, grid, (3, 3, 3), het.HET_F32)
    lib = het.load_library()
    need = int(lib.het_attn_route_workspace_bytes(ctypes.byref(shape)))
    assert 0 < need <= ws.numel()
    st = lib.het_attn_route(ctypes.byref(shape), u_gpu.data_ptr(), het.HET_TOP_RHO, float(rho), ctypes.byref(rs),
                            ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == het.HET_OK
    torch.cuda.synchronize()
    return dict(mask=bufs[0].cpu().numpy(), dense_idx=bufs[1].cpu().numpy(), local_idx=bufs[2].cpu().numpy(),
                counts=bufs[3].cpu().numpy(), thresh=bufs[4].cpu().numpy())


def test_route_workspace_reused_and_dirty(oracle_mod):
    """The workspace needs no clearing: filled with 0xff, with random bytes,
    and reused call after call (each call marks its barriers with a value of
    its own), every route is the oracle's."""
    import torch
    rng = np.random.default_rng(11)
    n = 21 * 30 * 52
    ws = torch.full((2 * 1024 * 1024,), 255, dtype=torch.uint8, device="cuda")
    for it, fill in enumerate(["ff", "random", "reuse", "reuse"]):
        if fill == "random":
            ws.copy_(torch.from_numpy(rng.integers(0, 256, ws.numel(), dtype=np.uint8)).cuda())
        u = rng.standard_normal((2, n)).astype(np.float32)
        rho = (0.2, 0.05, 0.6, 1.0 / n)[it]
        log(f"[route] workspace {fill} rho={rho}")
        g = route_via_abi(torch.from_numpy(u).cuda(), (21, 30, 52), rho, ws)
        assert_route_equal(g, oracle_mod.route_top_rho(u, rho))


@pytest.mark.parametrize("k", [2048, 4096, 4097, 6143, 12287])
def test_route_k_at_workgroup_edges(oracle_mod, k):
    """K at and next to multiples of the 2048 tokens a workgroup holds, with
    every u equal (the dense tokens are the first K by index, so the tie rule
    crosses workgroups) and with 40 distinct values."""
    n = 12288
    rng = np.random.default_rng(k)
    u = np.empty((2, n), np.float32)
    u[0] = 0.5
    u[1] = np.round(rng.random(n) * 39) / 39
    rho = (k - 0.25) / n  # floor(rho * n + 1/2) = k
    log(f"[route] N={n} K={k}")
    g = run_top_rho(oracle_mod, u, (1, 1, n), rho)
    assert g["counts"][0, 0] == k
    assert g["dense_idx"][0, :k].tolist() == list(range(k))


def test_route_many_workgroups_special_values(oracle_mod):
    """NaN (read as +inf), +-inf and -0 (read as +0) at a size routed by 12
    workgroups; keys one ulp apart in the other sample (one 1-bit digit)."""
    n = 24000
    rng = np.random.default_rng(21)
    u = rng.standard_normal((2, n)).astype(np.float32)
    u[0, rng.choice(n, 50, replace=False)] = np.nan
    u[0, rng.choice(n, 50, replace=False)] = np.inf
    u[0, rng.choice(n, 50, replace=False)] = -np.inf
    u[0, rng.choice(n, 300, replace=False)] = 0.0
    u[0, rng.choice(n, 300, replace=False)] = -0.0
    a = np.float32(1.0)
    u[1] = np.where(rng.random(n) < 0.5, a, np.nextafter(a, np.float32(2.0)))
    for rho in (0.001, 0.2, 0.5, 0.999):
        log(f"[route] N={n} special values rho={rho}")
        run_top_rho(oracle_mod, u, (1, 1, n), rho)


def test_route_largest_launch(oracle_mod):
    """1024 workgroups in one launch: 8 samples of 262144 tokens (128
    workgroups each), the most the several-workgroup route takes."""
    n = 64 * 64 * 64
    rng = np.random.default_rng(31)
    u = rng.lognormal(0.0, 1.0, (8, n)).astype(np.float32)
    log(f"[route] B=8 N={n}")
    run_top_rho(oracle_mod, u, (64, 64, 64), 0.2)


def top_bins(u, rho):
    """Keys (the order-preserving map of float32 u) that share the K-th
    largest key's top 11 and top 22 bits, per sample."""
    b = np.ascontiguousarray(u, np.float32).view(np.uint32).astype(np.uint64)
    b = np.where(np.isnan(u), np.uint64(0x7fc00000), b)
    keys = np.where(b >> 31, ~b & 0xffffffff, b | 0x80000000)
    out = []
    for row in keys:
        k = int(np.floor(rho * row.size + 0.5))
        kth = np.sort(row)[::-1][k - 1]
        out.append((int(np.sum(row >> 21 == kth >> 21)), int(np.sum(row >> 10 == kth >> 10))))
    return out


@pytest.mark.parametrize("case", ["bin_4096", "bin_4097", "narrow", "wide", "tied", "lists_whole_or_empty"])
def test_route_selection_paths(oracle_mod, case):
    """The several-workgroup top-rho select gathers the keys of the K-th
    key's bin as candidates once at most 4096 share its top 11 bits, else
    its top 22 bits, else it exchanges a third histogram and the counts.
    Each case is built for one of those paths (checked on the host) at its
    boundary: exactly 4096 and 4097 keys in the first bin, u spread wide
    (Gaussian) or narrow (within one octave), all tied, and candidate lists
    that are a whole workgroup's 2048 tokens or empty (4096 keys in all)."""
    rng = np.random.default_rng(77)
    n = 16384
    if case in ("bin_4096", "bin_4097"):
        m = 4096 if case == "bin_4096" else 4097
        # m keys in [1, 1.25) (one top-11 bin), the rest in [4, 5), shuffled
        u = np.where(np.arange(n) < m, 1.0 + 0.25 * rng.random(n), 4.0 + rng.random(n)).astype(np.float32)
        u = u[rng.permutation(n)][None]
        rho = (n - m + 100 - 0.25) / n
        want = "first" if m <= 4096 else "second"
    elif case == "narrow":
        n = 32760
        u = (1.0 + 0.01 * rng.standard_normal((2, n))).astype(np.float32)
        rho, want = 0.2, "second"
    elif case == "wide":
        n = 32760
        u = rng.standard_normal((2, n)).astype(np.float32)
        rho, want = 0.2, "first"
    elif case == "tied":
        u = np.full((1, n), 0.75, np.float32)
        u[0, rng.choice(n, 50, replace=False)] = 3.0
        rho, want = 0.3, "histograms"
    else:
        # tokens 2048..4095 and 8192..10239 hold the bin's keys (two whole
        # workgroups' lists), the others lie above or below it
        u = np.where(rng.random(n) < 0.5, 0.1 * rng.random(n), 8.0 + rng.random(n)).astype(np.float32)
        u[2048:4096] = 1.0 + 0.2 * rng.random(2048)
        u[8192:10240] = 1.0 + 0.2 * rng.random(2048)
        u = u[None]
        above = int(np.sum(u >= 8.0))
        rho = (above + 1000 - 0.25) / n
        want = "first"
    for first, second in top_bins(u, rho):
        got = "first" if first <= 4096 else ("second" if second <= 4096 else "histograms")
        assert got == want, (first, second)
    log(f"[route] selection path {case} B={u.shape[0]} N={u.shape[1]} rho={rho:.4f}")
    run_top_rho(oracle_mod, u, (1, 1, u.shape[1]), rho)


def test_route_selection_paths_mixed_in_one_launch(oracle_mod):
    """Samples of one launch on different selection paths at once: all tied
    (three histogram exchanges and the counts), spread wide (candidates after
    the first exchange) and narrow (candidates after the second)."""
    rng = np.random.default_rng(79)
    n = 24576
    u = np.empty((3, n), np.float32)
    u[0] = 0.5
    u[0, rng.choice(n, 40, replace=False)] = 2.0
    u[1] = rng.standard_normal(n)
    u[2] = 1.0 + 0.01 * rng.standard_normal(n)
    rho = 0.25
    paths = []
    for first, second in top_bins(u, rho):
        paths.append("first" if first <= 4096 else ("second" if second <= 4096 else "histograms"))
    assert paths == ["histograms", "first", "second"], paths
    log(f"[route] mixed selection paths B=3 N={n}")
    run_top_rho(oracle_mod, u, (1, 1, n), rho)
