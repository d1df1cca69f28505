"""Seeded synthetic inputs for uncertainty-routed heterogeneous attention.

This module only draws inputs; it holds none of the method's arithmetic.  Both
the HIP path (through its tests and the benchmark) and the CPU oracle receive
the very same arrays from here.

The shapes follow the latent grids of the two video models the HetA-DiT paper
evaluates ("Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion", §4 Evaluation Setting: 81x480x832 for Wan2.1, 121x704x1280 for
Wan2.2).  Trained activations and uncertainty maps are not available, so
N(0,1) Q/K/V and synthetic uncertainty fields stand in for them:

* ``iid``       u ~ U[0, 1) per token;
* ``lognormal`` u = Gaussian-smoothed exp(z), z ~ N(0, 1) on the (T, H, W)
  grid, sigma = 2 tokens, truncated at 3 sigma, reflecting borders;
* ``blobs``     three ellipsoidal blobs with Gaussian fall-off whose centres
  drift one token per frame (reflecting at the frame border), plus U[0, 0.1)
  noise -- concentrated difficulty that stresses load balance;
* ``ties``      u quantised to multiples of 1/16 (many equal values);
* ``equal``     every u the same.

Seeds: numpy ``Generator(PCG64(1000*config_id + tensor_id))`` with tensor ids
Q=1, K=2, V=3, u of sample b = 4 + b.  Q/K/V are drawn in float32 and, for
bf16 workloads, rounded to bf16 (round to nearest even); the returned float32
arrays then hold exactly the bf16 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    batch: int
    heads: int
    head_dim: int
    grid: tuple          # (T, H, W)
    window: tuple        # (wt, wh, ww), odd
    rho: float
    dtype: str           # "bf16" or "f32"
    u_kind: str
    scale: float = 0.0   # <= 0 means 1/sqrt(head_dim)
    extra: dict = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / float(np.sqrt(self.head_dim))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 64, (4, 8, 8), (3, 3, 3), 0.25, "f32", "iid"),
    "wan13b": Workload("wan13b", 2, 1, 12, 128, (21, 30, 52), (3, 7, 7), 0.2, "bf16", "lognormal"),
    "wan5b": Workload("wan5b", 3, 2, 24, 128, (31, 22, 40), (3, 7, 7), 0.2, "bf16", "lognormal"),
    "long": Workload("long", 5, 1, 12, 128, (41, 30, 52), (3, 7, 7), 0.2, "bf16", "blobs"),
}

# rho sweep on the Wan2.1-1.3B layer shape, same seeded inputs as "wan13b".
RHO_SWEEP = (0.05, 0.1, 0.2, 0.4, 1.0)

# Local neighbourhoods of the paper's window ablation (Table 7; 11x11x11 is
# its default), on the same seeded inputs as the 3x7x7 workloads.
WINDOW_SWEEP = ((9, 9, 9), (11, 11, 11), (13, 13, 13))
WORKLOADS["wan13b_w11"] = WORKLOADS["wan13b"].with_(name="wan13b_w11", window=(11, 11, 11))
WORKLOADS["wan5b_w11"] = WORKLOADS["wan5b"].with_(name="wan5b_w11", window=(11, 11, 11))


def _rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * config_id + tensor_id))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def make_qkv(w: Workload):
    """Q, K, V as float32 arrays [B, N, heads, D] (bf16-exact for bf16 workloads)."""
    shape = (w.batch, w.n_tokens, w.heads, w.head_dim)
    out = []
    for tid in (1, 2, 3):
        x = _rng(w.config_id, tid).standard_normal(shape, dtype=np.float32)
        if w.dtype == "bf16":
            x = round_to_bf16(x)
        out.append(x)
    return tuple(out)


def _lognormal_field(rng, grid):
    from scipy.ndimage import gaussian_filter
    z = rng.standard_normal(grid)
    return gaussian_filter(np.exp(z), sigma=2.0, mode="reflect", truncate=3.0)


def _blob_field(rng, grid):
    T, H, W = grid
    field_ = np.zeros(grid, np.float64)
    yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    for _ in range(3):
        ah, aw = rng.uniform(3.0, 6.0), rng.uniform(4.0, 9.0)
        cy, cx = rng.uniform(0, H - 1), rng.uniform(0, W - 1)
        theta = rng.uniform(0.0, 2.0 * np.pi)
        vy, vx = np.sin(theta), np.cos(theta)
        for t in range(T):
            field_[t] += np.exp(-0.5 * (((yy - cy) / ah) ** 2 + ((xx - cx) / aw) ** 2))
            cy, cx = cy + vy, cx + vx
            if cy < 0 or cy > H - 1:
                vy = -vy
                cy = min(max(cy, 0.0), H - 1.0)
            if cx < 0 or cx > W - 1:
                vx = -vx
                cx = min(max(cx, 0.0), W - 1.0)
    field_ += rng.uniform(0.0, 0.1, grid)
    return field_


def make_u(w: Workload, kind: str | None = None) -> np.ndarray:
    """Uncertainty u as float32 [B, N]; sample b uses seed tensor id 4 + b."""
    kind = kind or w.u_kind
    rows = []
    for b in range(w.batch):
        rng = _rng(w.config_id, 4 + b)
        if kind == "iid":
            x = rng.random(w.n_tokens)
        elif kind == "lognormal":
            x = _lognormal_field(rng, w.grid).reshape(-1)
        elif kind == "blobs":
            x = _blob_field(rng, w.grid).reshape(-1)
        elif kind == "ties":
            x = np.floor(rng.random(w.n_tokens) * 16.0) / 16.0
        elif kind == "equal":
            x = np.full(w.n_tokens, 0.5)
        else:
            raise ValueError(f"unknown u kind {kind!r}")
        rows.append(np.asarray(x, dtype=np.float32))
    return np.ascontiguousarray(np.stack(rows))


def dense_count(n_tokens: int, rho: float) -> int:
    """Number of dense tokens at dense fraction rho: round half up of rho*N."""
    return int(min(max(np.floor(rho * n_tokens + 0.5), 0), n_tokens))


def effective_flops(w: Workload, dense_counts=None) -> float:
    """FLOPs the routing requires ([HetA §3.2.2 Eq. 14] with 2 flops per
    multiply-add for QK^T and for PV): 4*D*heads*sum_b(K_b*N + (N-K_b)*M)."""
    N = w.n_tokens
    T, H, W = w.grid
    M = min(w.window[0], T) * min(w.window[1], H) * min(w.window[2], W)
    if dense_counts is None:
        dense_counts = [dense_count(N, w.rho)] * w.batch
    return float(sum(4.0 * w.head_dim * w.heads * (k * N + (N - k) * M) for k in dense_counts))
