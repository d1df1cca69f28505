"""Calls on a side stream.

The binding allocates a call's outputs and workspace under the stream the
call runs on, so PyTorch's caching allocator does not hand a workspace freed
at the call's return to work on another stream while the call's kernels
still read it.  Route, forward (with the rows' LSE) and backward issued on a
side stream of the default priority, while the current stream allocates and
writes fresh tensors, must give bit-identical results to the same calls on
the current stream (the kernels are deterministic).
"""
import numpy as np
import pytest

import uncertainty_routed_heterogeneous_amd as het
import workloads as W
from gpu_util import log, to_gpu

pytestmark = pytest.mark.gpu


def test_side_stream_matches_current_stream():
    import torch
    w = W.Workload("streams", 990, 2, 3, 128, (6, 10, 20), (3, 7, 7), 0.3, "bf16", "lognormal")
    q, k, v = W.make_qkv(w)
    u = W.make_u(w)
    dout = W.round_to_bf16(np.random.default_rng(3).standard_normal(q.shape).astype(np.float32))
    qg, kg, vg, dg = (to_gpu(x, "bf16") for x in (q, k, v, dout))
    ug = to_gpu(u.astype(np.float32))
    log("[streams] current stream")
    r0 = het.route(ug, w.grid, w.window, w.heads, w.head_dim, torch.bfloat16, rho=w.rho)
    o0, lse0 = het.forward(qg, kg, vg, r0, return_lse=True)
    g0 = het.backward(qg, kg, vg, r0, o0, dg, lse=lse0)
    torch.cuda.synchronize()

    log("[streams] side stream")
    s = torch.cuda.Stream()  # default priority
    r1 = het.route(ug, w.grid, w.window, w.heads, w.head_dim, torch.bfloat16, rho=w.rho, stream=s)
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(32)]
    o1, lse1 = het.forward(qg, kg, vg, r1, return_lse=True, stream=s)
    junk += [torch.full((1 << 22,), -3.0, device="cuda") for _ in range(16)]
    g1 = het.backward(qg, kg, vg, r1, o1, dg, lse=lse1, stream=s)
    junk += [torch.full((1 << 24,), 5.0, device="cuda") for _ in range(4)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(r0.mask, r1.mask) and torch.equal(r0.dense_idx, r1.dense_idx)
    assert torch.equal(o0, o1) and torch.equal(lse0, lse1)
    for name, a, b in zip(("dQ", "dK", "dV"), g0, g1):
        assert torch.equal(a, b), name
