"""Helpers for the GPU parity tests: move seeded numpy inputs to the GPU,
call the library through its binding, bring results back, and compare
against the oracle with the tolerances the tests state."""
from __future__ import annotations

import sys

import numpy as np

import uncertainty_routed_heterogeneous_amd as het


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(name: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def to_gpu(x: np.ndarray, dtype_name: str | None = None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype_name is not None:
        t = t.to(torch_dtype(dtype_name))
    return t.cuda()


def gpu_route(u: np.ndarray, grid, window, heads, head_dim, dtype_name, rho=None, c=None):
    import torch
    r = het.route(to_gpu(u.astype(np.float32)), grid, window, heads, head_dim,
                  torch_dtype(dtype_name), rho=rho, c=c)
    torch.cuda.synchronize()
    return r


def route_to_numpy(r):
    return dict(mask=r.mask.cpu().numpy(), dense_idx=r.dense_idx.cpu().numpy(),
                local_idx=r.local_idx.cpu().numpy(), counts=r.counts.cpu().numpy(),
                thresh=r.thresh.cpu().numpy())


def assert_route_equal(g: dict, o, exact_thresh: bool = True) -> None:
    """Bit-exact comparison of a GPU route with the oracle's (the threshold
    too, unless it comes from an fp64 sum taken in a different order)."""
    np.testing.assert_array_equal(g["counts"], o.counts)
    np.testing.assert_array_equal(g["mask"], o.mask)
    np.testing.assert_array_equal(g["dense_idx"], o.dense_idx)
    np.testing.assert_array_equal(g["local_idx"], o.local_idx)
    if exact_thresh:
        np.testing.assert_array_equal(g["thresh"], o.thresh)


def gpu_forward(q, k, v, r, dtype_name, scale=None, prefill=None):
    """het.forward on the GPU; with prefill, the output tensor starts filled
    with that value (NaN shows a row the kernels did not write)."""
    import torch
    qg, kg, vg = to_gpu(q, dtype_name), to_gpu(k, dtype_name), to_gpu(v, dtype_name)
    out = torch.full_like(qg, prefill) if prefill is not None else None
    o = het.forward(qg, kg, vg, r, scale=scale, out=out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


# Tolerances for outputs against the fp64 oracle: bf16 inputs with fp32
# accumulation (probabilities rounded to bf16 before P*V) and fp32 inputs.
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3), "f32": dict(max_abs=1e-5, mean_abs=1e-6)}


def assert_close(got: np.ndarray, ref: np.ndarray, dtype_name: str, what: str = "") -> dict:
    err = np.abs(got.astype(np.float64) - ref)
    stats = dict(max_abs=float(err.max()) if err.size else 0.0,
                 mean_abs=float(err.mean()) if err.size else 0.0)
    tol = TOL[dtype_name]
    log(f"  {what} max_abs={stats['max_abs']:.3e} mean_abs={stats['mean_abs']:.3e} "
        f"(tol {tol['max_abs']:.0e}/{tol['mean_abs']:.0e})")
    assert stats["max_abs"] <= tol["max_abs"], f"{what}: max abs error {stats['max_abs']}"
    assert stats["mean_abs"] <= tol["mean_abs"], f"{what}: mean abs error {stats['mean_abs']}"
    return stats
