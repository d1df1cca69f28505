"""GPU backward pass (het_attn_backward) against the fp64 oracle.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): the routed layer (§3.2.2 Eq. 13 over §3.1.1 Eqs. 2-3)
differentiated with the route held fixed, as the second training stage needs
(§4, Training Setting).

Errors are taken relative to the largest magnitude of each reference
gradient tensor G: max |got - ref| / max |G| and mean |got - ref| / max |G|.
Bounds: bf16 2e-2 / 2e-3 (inputs exact, P and dS rounded to bf16 as MFMA
operands, outputs rounded to bf16: a few 2^-8 relative per term), fp32
1e-5 / 1e-6.  Small cases compare every element of dQ, dK and dV; the full
Wan2.1-1.3B, Wan2.2-5B and long-video shapes compare sampled dQ rows and
the dK, dV rows of sampled keys (the oracle sums each key's gradient over
every row that sees it), plus identities that hold at any size: the key
gradients of a (sample, head) sum to zero and the value gradients sum to
the sum of dO.
"""
import numpy as np
import pytest

import uncertainty_routed_heterogeneous_amd as het
import workloads as W
from gpu_util import gpu_route, log, to_gpu, torch_dtype

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-6)}


def rel_check(got, ref, dtype, what):
    scale = float(np.abs(ref).max()) or 1.0
    err = np.abs(got.astype(np.float64) - ref) / scale
    mx, mean = float(err.max()), float(err.mean())
    tmax, tmean = TOL[dtype]
    log(f"  {what}: max {mx:.2e} mean {mean:.2e} of max|ref| {scale:.3e} (tol {tmax:.0e}/{tmean:.0e})")
    assert np.isfinite(got).all(), what
    assert mx <= tmax and mean <= tmean, what


def make_case(grid, heads, head_dim, dtype, batch=2, seed=0, window=(3, 7, 7), u_kind="iid"):
    w = W.Workload(f"bwd{seed}", 970 + seed, batch, heads, head_dim, tuple(grid), tuple(window), 0.3,
                   dtype, u_kind)
    q, k, v = W.make_qkv(w)
    rng = np.random.default_rng(4000 + seed)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    if dtype == "bf16":
        dout = W.round_to_bf16(dout)
    return w, q, k, v, dout, W.make_u(w)


def gpu_backward(w, q, k, v, dout, r, border="shift"):
    import torch
    t = lambda x: to_gpu(x, w.dtype)
    qg, kg, vg, dg = t(q), t(k), t(v), t(dout)
    o = het.forward(qg, kg, vg, r, border=border)
    dq, dk, dv = het.backward(qg, kg, vg, r, o, dg, border=border)
    torch.cuda.synchronize()
    return tuple(x.float().cpu().numpy() for x in (dq, dk, dv))


def full_check(oracle_mod, w, q, k, v, dout, r, what, border="shift"):
    log(f"[backward] {what} grid={w.grid} win={w.window} B={w.batch} H={w.heads} D={w.head_dim} "
        f"{w.dtype} border={border}")
    got = gpu_backward(w, q, k, v, dout, r, border)
    mask = r.mask.cpu().numpy()
    ref = oracle_mod.backward(q, k, v, dout, w.grid, w.window, w.softmax_scale, mask, border=border)
    for name, g, rf in zip(("dQ", "dK", "dV"), got, ref):
        rel_check(g, rf, w.dtype, f"{what} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("rho", [0.0, 0.3, 1.0])
def test_backward_small_grid(oracle_mod, dtype, head_dim, rho):
    # N = 1200: ragged query and key tiles in every axis, 38 dense blocks of 32.
    w, q, k, v, dout, u = make_case((6, 10, 20), 2, head_dim, dtype, seed=head_dim + int(10 * rho))
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, dtype, rho=rho)
    full_check(oracle_mod, w, q, k, v, dout, r, f"rho={rho}")


@pytest.mark.parametrize("window", [(1, 3, 3), (5, 9, 13), (3, 9, 25), (11, 11, 11)])
def test_backward_windows(oracle_mod, window):
    w, q, k, v, dout, u = make_case((15, 18, 29), 1, 128, "bf16", batch=1, seed=window[2], window=window)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", rho=0.2)
    full_check(oracle_mod, w, q, k, v, dout, r, f"window {window}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_cut_border(oracle_mod, dtype):
    w, q, k, v, dout, u = make_case((6, 10, 20), 2, 64, dtype, seed=31, window=(3, 7, 9))
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, dtype, rho=0.2)
    full_check(oracle_mod, w, q, k, v, dout, r, "cut border", border="cut")


@pytest.mark.parametrize("grid,window,head_dim", [
    ((9, 3, 5), (3, 3, 3), 64),      # 15 positions per frame: a 128-key block spans 9 frames
    ((3, 1, 200), (1, 1, 7), 128),   # one row per frame, 200 long
    ((2, 13, 70), (3, 7, 7), 128),   # rows longer than a key block; a column tile's queries span 17
    ((2, 13, 71), (3, 7, 7), 128),   # three ragged column groups, each tile's queries within 16 columns
])
def test_backward_key_block_layouts(oracle_mod, grid, window, head_dim):
    w, q, k, v, dout, u = make_case(grid, 2, head_dim, "bf16", batch=2, seed=61 + grid[2], window=window)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", rho=0.25)
    full_check(oracle_mod, w, q, k, v, dout, r, f"key blocks {grid}")


def test_backward_mean_std_and_swapped_routes(oracle_mod):
    import torch
    w, q, k, v, dout, u = make_case((6, 10, 20), 2, 128, "bf16", seed=41, u_kind="lognormal")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", c=0.9)
    full_check(oracle_mod, w, q, k, v, dout, r, "mean-std route")
    (rs,) = het.swap(r, 0.1, 5, 0, 3)
    torch.cuda.synchronize()
    full_check(oracle_mod, w, q, k, v, dout, rs, "swapped route")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_single_token(oracle_mod, dtype):
    w, q, k, v, dout, u = make_case((1, 1, 1), 1, 64, dtype, batch=1, seed=51, window=(3, 3, 3))
    for rho in (0.0, 1.0):
        r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, dtype, rho=rho)
        dq, dk, dv = gpu_backward(w, q, k, v, dout, r)
        # one key: P = 1, so dV = dO, and dS = P (dP - D) = 0 up to the two
        # fp32 sums for dP and D, so dQ = dK = 0 to that rounding
        np.testing.assert_allclose(dv, dout, rtol=0, atol=1e-6)
        tol = 1e-4 if dtype == "bf16" else 1e-5
        assert np.abs(dq).max() < tol and np.abs(dk).max() < tol


def sampled_keys(w, mask_b, rng, n_random=24):
    """Keys of one sample whose dK, dV rows are compared: the grid's corners
    and face centres, both ends of the first and last 128-key blocks, dense
    tokens with their next neighbours along each axis (keys seen by many
    dense rows and by the local rows around them), and random keys."""
    T, H, W_ = w.grid
    N = w.n_tokens
    tok = lambda t, y, x: (t * H + y) * W_ + x
    keys = [tok(t, y, x) for t in (0, T - 1) for y in (0, H - 1) for x in (0, W_ - 1)]
    keys += [tok(T // 2, H // 2, 0), tok(T // 2, H // 2, W_ - 1), tok(T // 2, 0, W_ // 2),
             tok(T // 2, H - 1, W_ // 2), tok(0, H // 2, W_ // 2), tok(T - 1, H // 2, W_ // 2)]
    keys += [0, 1, 127, 128, 129, 255, N - 1, N - 2, N - 128, N - 129]
    dense = np.nonzero(mask_b == 0)[0]
    for j in rng.choice(dense, min(6, dense.size), replace=False):
        t, y, x = j // (H * W_), (j // W_) % H, j % W_
        keys += [j, tok(t, y, min(x + 1, W_ - 1)), tok(t, min(y + 1, H - 1), x), tok(min(t + 1, T - 1), y, x)]
    keys += rng.choice(N, n_random, replace=False).tolist()
    return np.unique(np.array(keys, dtype=np.int64) % N)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,head", [("wan13b", 5), ("wan5b", 23), ("long", 0)])
def test_backward_full_size_sampled(oracle_mod, name, head):
    """The benchmark's training form at the full layer shapes (forward with
    the rows' LSE, backward given it), outputs prefilled with NaN so that an
    unwritten row shows: every element finite, dQ of sampled rows (all
    heads) and dK, dV of sampled keys (one head, summed by the oracle over
    every row that sees the key) element by element against the oracle."""
    import torch
    w = W.WORKLOADS[name]
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    dout = W.round_to_bf16(np.random.default_rng(77).standard_normal(q.shape).astype(np.float32))
    log(f"[backward] full size {name} B={w.batch} H={w.heads} N={w.n_tokens} rho={w.rho}")
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", rho=w.rho)
    qg, kg, vg, dg = (to_gpu(x, "bf16") for x in (q, k, v, dout))
    nan = lambda: torch.full_like(qg, float("nan"))
    o, lse = het.forward(qg, kg, vg, r, return_lse=True, out=nan())
    dq, dk, dv = het.backward(qg, kg, vg, r, o, dg, lse=lse, out=(nan(), nan(), nan()))
    torch.cuda.synchronize()
    for name_, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), f"{name} {name_}: an element is not finite (unwritten row?)"
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    mask = r.mask.cpu().numpy()
    B, N, H, D = w.batch, w.n_tokens, w.heads, w.head_dim
    rng = np.random.default_rng(8)
    rows, keys = [], []
    for b in range(B):
        dense = np.nonzero(mask[b] == 0)[0]
        local = np.nonzero(mask[b] == 1)[0]
        rows.append(b * N + np.unique(np.concatenate([rng.choice(dense, 16, replace=False),
                                                      rng.choice(local, 24, replace=False),
                                                      [dense[0], dense[-1], local[0], local[-1]]])))
        keys.append(b * N + sampled_keys(w, mask[b], rng))
    rows = np.concatenate(rows).astype(np.int64)
    keys = np.concatenate(keys).astype(np.int64)
    ref = oracle_mod.backward_dq_rows(q, k, v, dout, w.grid, w.window, w.softmax_scale, mask, rows)
    rel_check(dq.reshape(B * N, H, D)[rows], ref, "bf16", f"{name} dQ of {rows.size} sampled rows")
    log(f"  oracle dK, dV of {keys.size} keys, head {head}")
    rk, rv = oracle_mod.backward_kv_rows(q, k, v, dout, w.grid, w.window, w.softmax_scale, mask, keys,
                                         heads=[head])
    rel_check(dk.reshape(B * N, H, D)[keys][:, [head]], rk, "bf16", f"{name} dK of {keys.size} sampled keys")
    rel_check(dv.reshape(B * N, H, D)[keys][:, [head]], rv, "bf16", f"{name} dV of {keys.size} sampled keys")
    # sum identities over all keys of every head (float64 sums of the bf16 results)
    sk = dk.astype(np.float64).sum(axis=1)          # [B, heads, D]
    ak = np.abs(dk.astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(sk) <= 4e-3 * ak + 1e-6), float((np.abs(sk) / ak).max())
    sv = dv.astype(np.float64).sum(axis=1)
    so = dout.astype(np.float64).sum(axis=1)
    av = np.abs(dv.astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(sv - so) <= 4e-3 * av + 1e-3), float((np.abs(sv - so) / av).max())


LOG2E = 1.4426950408889634


@pytest.mark.parametrize("grid,window,head_dim,rho", [
    ((6, 10, 20), (3, 7, 7), 128, 0.3),
    ((6, 10, 20), (3, 7, 7), 64, 0.0),
    ((6, 10, 20), (3, 7, 7), 64, 1.0),
    ((2, 13, 70), (3, 7, 7), 128, 0.25),   # the dK/dV pass takes the local queries itself
    ((9, 3, 5), (3, 3, 3), 64, 0.4),
    ((4, 9, 40), (3, 7, 7), 128, 0.2),     # local kernel: one frame x 8 x-tiles
    ((4, 9, 14), (3, 7, 7), 128, 0.2),     # local kernel: two frames x 4 x-tiles
])
def test_forward_lse_and_backward_lse(oracle_mod, grid, window, head_dim, rho):
    """het_attn_forward_lse writes the same O as het_attn_forward and each row's
    log2-sum-exp (checked against the oracle's normaliser); het_attn_backward_lse
    given it returns exactly what het_attn_backward computes on its own."""
    import torch
    w, q, k, v, dout, u = make_case(grid, 2, head_dim, "bf16", batch=2, seed=91 + grid[2] + int(10 * rho),
                                    window=window)
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", rho=rho)
    qg, kg, vg, dg = (to_gpu(x, "bf16") for x in (q, k, v, dout))
    log(f"[lse] grid={grid} win={window} D={head_dim} rho={rho}")
    o = het.forward(qg, kg, vg, r)
    o2, lse = het.forward(qg, kg, vg, r, return_lse=True)
    g_ref = het.backward(qg, kg, vg, r, o, dg)
    g_lse = het.backward(qg, kg, vg, r, o2, dg, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    B, N, H = w.batch, w.n_tokens, w.heads
    mask = r.mask.cpu().numpy()
    ref = oracle_mod.row_lse(q, k, w.grid, w.window, w.softmax_scale, mask, np.arange(B * N))
    ref = ref.reshape(B, N, H).transpose(0, 2, 1) * LOG2E
    got = lse.cpu().numpy()
    err = np.abs(got - ref)
    log(f"  lse: max {err.max():.2e} mean {err.mean():.2e} (log2 units)")
    # scores from the bf16-rounded pre-scaled query: a few 2^-9 relative
    assert np.isfinite(got).all() and err.max() < 2e-2 and err.mean() < 2e-3
    for name, a, b in zip(("dQ", "dK", "dV"), g_ref, g_lse):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("router,border", [("mean_std", "shift"), ("top_rho", "cut")])
def test_lse_forms_other_routes_and_border(oracle_mod, router, border):
    """Dense counts unknown to the host (mean-std threshold: the merge of the
    dense kernel's split units runs over device-side counts) and the cut
    border: the forward's LSE against the oracle, the backward given it
    against the oracle's gradients."""
    import torch
    w, q, k, v, dout, u = make_case((6, 10, 20), 2, 128, "bf16", batch=2, seed=97, window=(3, 7, 9),
                                    u_kind="lognormal")
    r = (gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", c=0.9) if router == "mean_std"
         else gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", rho=0.2))
    qg, kg, vg, dg = (to_gpu(x, "bf16") for x in (q, k, v, dout))
    log(f"[lse] {router} border={border}")
    o, lse = het.forward(qg, kg, vg, r, return_lse=True, border=border)
    grads = het.backward(qg, kg, vg, r, o, dg, lse=lse, border=border)
    torch.cuda.synchronize()
    B, N, H = w.batch, w.n_tokens, w.heads
    mask = r.mask.cpu().numpy()
    ref = oracle_mod.row_lse(q, k, w.grid, w.window, w.softmax_scale, mask, np.arange(B * N), border=border)
    err = np.abs(lse.cpu().numpy() - ref.reshape(B, N, H).transpose(0, 2, 1) * LOG2E)
    log(f"  lse: max {err.max():.2e} mean {err.mean():.2e} (log2 units)")
    assert err.max() < 2e-2 and err.mean() < 2e-3
    refs = oracle_mod.backward(q, k, v, dout, w.grid, w.window, w.softmax_scale, mask, border=border)
    for name, g, rf in zip(("dQ", "dK", "dV"), grads, refs):
        rel_check(g.float().cpu().numpy(), rf, "bf16", f"{router} {border} {name}")


def test_lse_forms_full_size():
    """Wan-1.3B shape: the backward given the forward's LSE equals the backward
    that computes it (the same kernels produce the same statistics)."""
    import torch
    w = W.WORKLOADS["wan13b"]
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    dout = W.round_to_bf16(np.random.default_rng(78).standard_normal(q.shape).astype(np.float32))
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "bf16", rho=w.rho)
    qg, kg, vg, dg = (to_gpu(x, "bf16") for x in (q, k, v, dout))
    log(f"[lse] full size {w.name}")
    o, lse = het.forward(qg, kg, vg, r, return_lse=True)
    g_ref = het.backward(qg, kg, vg, r, o, dg)
    g_lse = het.backward(qg, kg, vg, r, o, dg, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()
    for name, a, b in zip(("dQ", "dK", "dV"), g_ref, g_lse):
        assert torch.equal(a, b), name


def test_lse_forms_reject_fp32_and_bad_lse():
    import torch
    w, q, k, v, dout, u = make_case((3, 4, 5), 1, 64, "f32", batch=1, seed=5, window=(3, 3, 3))
    r = gpu_route(u, w.grid, w.window, w.heads, w.head_dim, "f32", rho=0.3)
    qg, kg, vg = (to_gpu(x, "f32") for x in (q, k, v))
    with pytest.raises(het.HetAttnError):
        het.forward(qg, kg, vg, r, return_lse=True)
    qb, kb, vb, db = (to_gpu(x, "bf16") for x in (q, k, v, dout))
    o, lse = het.forward(qb, kb, vb, r, return_lse=True)
    with pytest.raises(ValueError):
        het.backward(qb, kb, vb, r, o, db, lse=lse[:, :, :-1].contiguous())
    torch.cuda.synchronize()
