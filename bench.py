#!/usr/bin/env python3
"""Benchmark of one uncertainty-routed heterogeneous attention layer on one
MI355X.

A step is one pass of the whole layer over one batch of synthetic inputs
already resident in HBM: threshold + mask + compaction (het_attn_route), the
local 3D-window rows (het_attn_local) and the gathered dense rows
(het_attn_dense) -- i.e. het_attn_route + het_attn_forward, issued as its two
halves so that HIP events can time the dense kernel by itself inside the
timed region.  Default workload: the Wan2.1-1.3B-shaped layer (B=1, 12
heads, head_dim 128, 21x30x52 latent grid, rho = 0.2, 3x7x7 window).

Prints ONE JSON line on stdout.  Extra detail goes to stderr.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): effective FLOPs follow the cost model of §3.2.2 Eq. 14.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/attn layer + effective TFLOP/s at rho=0.2 (Wan-1.3B shape); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
DENSE_KERNEL_SOURCES = ("uncertainty_routed_heterogeneous_amd/csrc/dense.hip",
                        "uncertainty_routed_heterogeneous_amd/csrc/common.hpp")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "dense_bf16_wan13b_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(dense_launch_units: float):
    """HBM bytes per dense launch from the committed counter summary, if it
    was taken on the current dense kernel source; else None."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(DENSE_KERNEL_SOURCES):
        return None
    return float(m_bytes.group(1))


class Layer:
    """Pre-built ctypes arguments for one workload, so the timed loop issues
    three library calls per step and nothing else."""

    def __init__(self, het, w, q, k, v, u, rho, router="top_rho", border="shift"):
        import torch
        self.het, self.lib, self.w = het, het.load_library(), w
        B, N = w.batch, w.n_tokens
        dev = q.device
        self.q, self.k, self.v, self.u = q, k, v, u
        self.o = torch.empty_like(q)
        self.mask = torch.empty((B, N), dtype=torch.uint8, device=dev)
        self.didx = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.lidx = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.counts = torch.empty((B, 2), dtype=torch.int32, device=dev)
        self.thresh = torch.empty((B,), dtype=torch.float64, device=dev)
        self.shape = het.make_shape(B, w.heads, w.head_dim, w.grid, w.window, het.HET_BF16, border=border)
        self.router = router
        self.rs = het.RouteStruct(self.mask.data_ptr(), self.didx.data_ptr(), self.lidx.data_ptr(),
                                  self.counts.data_ptr(), self.thresh.data_ptr(), -1)
        self.rho = float(rho)
        self.stream = torch.cuda.current_stream().cuda_stream
        ws = het.workspace_bytes(self.shape)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.ws_bytes = ws
        rws = int(self.lib.het_attn_route_workspace_bytes(ctypes.byref(self.shape)))
        self.rws = torch.empty(max(rws, 1), dtype=torch.uint8, device=dev)
        self.rws_bytes = rws
        self.args = (ctypes.byref(self.shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                     ctypes.byref(self.rs), self.o.data_ptr(), self.ws.data_ptr(), ws, self.stream)

    def route(self):
        if self.router == "random":
            st = self.lib.het_attn_route_random(ctypes.byref(self.shape), self.rho, 12345, 0, 0, 1,
                                                ctypes.byref(self.rs), self.stream)
        else:
            mode = self.het.HET_UNIFORM if self.router == "uniform" else self.het.HET_TOP_RHO
            st = self.lib.het_attn_route(ctypes.byref(self.shape), self.u.data_ptr(), mode, self.rho,
                                         ctypes.byref(self.rs), self.rws.data_ptr(), self.rws_bytes,
                                         self.stream)
        if st != 0:
            raise self.het.HetAttnError(st, "route (" + self.router + ")")

    def local(self):
        st = self.lib.het_attn_local(*self.args)
        if st != 0:
            raise self.het.HetAttnError(st, "het_attn_local")

    def dense(self):
        st = self.lib.het_attn_dense(*self.args)
        if st != 0:
            raise self.het.HetAttnError(st, "het_attn_dense")


def window_lengths(S: int, k: int, cut: bool):
    """Keys of the window along one axis for every position (shifted windows
    hold min(k, S); cut windows lose the positions past the border)."""
    import numpy as np
    pos = np.arange(S)
    if not cut:
        return np.full(S, min(k, S))
    h = (k - 1) // 2
    return np.minimum(pos + h + 1, S) - np.maximum(pos - h, 0)


def effective_flops_routed(w, mask, border: str) -> float:
    """4*D*heads*(sum of dense keys + sum of local window keys) for the route
    `mask` ([B, N], 1 = local): Eq. 14's terms, with the window size of each
    local token (constant M for shifted windows)."""
    import numpy as np
    T, H, Wd = w.grid
    cut = border == "cut"
    M = (window_lengths(T, w.window[0], cut)[:, None, None] * window_lengths(H, w.window[1], cut)[None, :, None]
         * window_lengths(Wd, w.window[2], cut)[None, None, :]).reshape(-1).astype(np.float64)
    total = 0.0
    for b in range(mask.shape[0]):
        local = mask[b] != 0
        total += float((~local).sum()) * w.n_tokens + float(M[local].sum())
    return 4.0 * w.head_dim * w.heads * total


def time_layer(layer, steps: int, warmup: int, scrub=None):
    """Warm up, then time exactly `steps` steps; per-kernel times come from
    events recorded between the launches on the same stream.  With `scrub`
    (a device tensor), every step is preceded, outside the events, by a write
    of the whole tensor, which evicts L2 and the last-level cache (cold
    timing)."""
    import torch
    for _ in range(warmup):
        layer.route(); layer.local(); layer.dense()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[E(), E(), E(), E()] for _ in range(steps)]
    start, end = E(), E()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(steps):
        if scrub is not None:
            scrub.fill_(s)
        ev[s][0].record(); layer.route()
        ev[s][1].record(); layer.local()
        ev[s][2].record(); layer.dense()
        ev[s][3].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    per = [[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in ev]
    mean = lambda xs: sum(xs) / len(xs)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    step = [sum(p) for p in per]
    return dict(ms_per_step=total_ms / steps, wall_ms_per_step=1e3 * wall / steps,
                route_ms=mean([p[0] for p in per]), local_ms=mean([p[1] for p in per]),
                dense_ms=mean([p[2] for p in per]),
                step_ms_median=med(step), route_ms_median=med([p[0] for p in per]),
                local_ms_median=med([p[1] for p in per]), dense_ms_median=med([p[2] for p in per]))


def time_swap(layer, ratio: float, n_blocks: int, iters: int, warmup: int = 3):
    """Median time of one het_attn_swap launch that makes the routes of
    n_blocks blocks from the layer's route (already computed)."""
    import torch
    het, w = layer.het, layer.w
    B, N = w.batch, w.n_tokens
    dev = layer.mask.device
    bufs = [torch.empty((n_blocks, B, N), dtype=torch.uint8, device=dev),
            torch.empty((n_blocks, B, N), dtype=torch.int32, device=dev),
            torch.empty((n_blocks, B, N), dtype=torch.int32, device=dev),
            torch.empty((n_blocks, B, 2), dtype=torch.int32, device=dev),
            torch.empty((n_blocks, B), dtype=torch.float64, device=dev)]
    out = het.RouteStruct(*[b.data_ptr() for b in bufs], -1)

    def launch(step):
        st = layer.lib.het_attn_swap(ctypes.byref(layer.shape), ctypes.byref(layer.rs), ratio, 12345,
                                     step, 0, n_blocks, ctypes.byref(out), layer.stream)
        if st != 0:
            raise het.HetAttnError(st, "het_attn_swap")

    layer.route()
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(E(), E()) for _ in range(iters)]
    for i, (a, b) in enumerate(ev):
        a.record(); launch(i); b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2]


def time_backward(layer, iters: int, warmup: int = 2, with_lse: bool = True):
    """Median time of one backward call on the layer's route and output, with
    a seeded dO: het_attn_backward_lse given the rows' LSE that
    het_attn_forward_lse wrote (with_lse), else het_attn_backward, which
    computes the LSE itself.  Per-kernel split from events is not possible
    inside one call, so only the whole call is timed here."""
    import torch
    het, w = layer.het, layer.w
    g = torch.Generator(device="cuda").manual_seed(77)
    dout = torch.randn(layer.q.shape, generator=g, device="cuda", dtype=torch.float32).to(layer.q.dtype)
    dq, dk, dv = (torch.empty_like(layer.q) for _ in range(3))
    ws_n = int(layer.lib.het_attn_backward_workspace_bytes(ctypes.byref(layer.shape)))
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    lse = torch.empty((w.batch, w.heads, w.n_tokens), dtype=torch.float32, device="cuda")
    layer.route()
    st = layer.lib.het_attn_forward_lse(*layer.args[:6], lse.data_ptr(), *layer.args[6:])
    if st != 0:
        raise het.HetAttnError(st, "het_attn_forward_lse")

    def call():
        if with_lse:
            st = layer.lib.het_attn_backward_lse(ctypes.byref(layer.shape), layer.q.data_ptr(), layer.k.data_ptr(),
                                                 layer.v.data_ptr(), ctypes.byref(layer.rs), layer.o.data_ptr(),
                                                 dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                                 dv.data_ptr(), ws.data_ptr(), ws_n, layer.stream)
        else:
            st = layer.lib.het_attn_backward(ctypes.byref(layer.shape), layer.q.data_ptr(), layer.k.data_ptr(),
                                             layer.v.data_ptr(), ctypes.byref(layer.rs), layer.o.data_ptr(),
                                             dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                             ws.data_ptr(), ws_n, layer.stream)
        if st != 0:
            raise het.HetAttnError(st, "het_attn_backward" + ("_lse" if with_lse else ""))

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [(E(), E()) for _ in range(iters)]
    for a, b in ev:
        a.record(); call(); b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, u, rho, stride: int):
    """The fp64 oracle on the host cores, on a bounded sample of the same
    layer: the full route (timed by itself), then every `stride`-th dense and
    local row of the layer (all heads), timed by itself; the rate is the
    sample's effective FLOPs over the route and forward seconds."""
    import numpy as np
    import oracle
    import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    r = oracle.route_top_rho(u, rho)
    t_route = time.perf_counter() - t0
    rows = []
    n_dense = n_local = 0
    for b in range(w.batch):
        d = r.dense_idx[b, : r.counts[b, 0]][::stride]
        l = r.local_idx[b, : r.counts[b, 1]][::stride]
        n_dense += d.size
        n_local += l.size
        rows.append(b * w.n_tokens + np.concatenate([d, l]).astype(np.int64))
    t1 = time.perf_counter()
    oracle.attend_rows(q, k, v, w.grid, w.window, w.softmax_scale, r.mask, np.concatenate(rows),
                       nthreads=threads)
    t_fwd = time.perf_counter() - t1
    sec = t_route + t_fwd
    T, H, Wd = w.grid
    M = min(w.window[0], T) * min(w.window[1], H) * min(w.window[2], Wd)
    flop = 4.0 * w.head_dim * w.heads * (n_dense * w.n_tokens + n_local * M)
    return {"value": round(flop / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(), "route_s": round(t_route, 3), "forward_s": round(t_fwd, 2),
            "sample": (f"{w.name}: the full route of {w.batch}x{w.n_tokens} tokens ({t_route:.2f} s) plus every "
                       f"{stride}th dense and local row ({n_dense} dense, {n_local} local rows, all {w.heads} "
                       f"heads; {t_fwd:.1f} s) in fp64 on {threads} threads; effective FLOPs of the sample per "
                       f"second; the whole layer would take about "
                       f"{t_route + W.effective_flops(w.with_(rho=rho)) / (flop / t_fwd):.0f} s at this rate")}


def run_sweep(het, W, torch, main_inputs, steps: int, warmup: int):
    """Warm timings (medians of `steps` steps after `warmup`) of the rho sweep
    and the window ablation on the Wan-1.3B shape and of the other workloads
    at their own rho: the inputs of each distinct workload are drawn once
    (the Wan-1.3B ones are the main run's).  A compact row per config."""
    cases = ([("wan13b", r, None) for r in W.RHO_SWEEP] +
             [("wan13b", None, win) for win in W.WINDOW_SWEEP] +
             [("wan5b", None, None), ("wan5b", None, (11, 11, 11)), ("long", None, None)])
    rows = []
    cache = {"wan13b": main_inputs}
    to_bf16 = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    for name, r, win in cases:
        w = W.WORKLOADS[name]
        if name not in cache:
            cache.clear()
            cache["wan13b"] = main_inputs
            qn, kn, vn = W.make_qkv(w)
            cache[name] = (to_bf16(qn), to_bf16(kn), to_bf16(vn), torch.from_numpy(W.make_u(w)).cuda())
            del qn, kn, vn
        q, k, v, u = cache[name]
        if win is not None:
            w = w.with_(window=win)
        rho = w.rho if r is None else r
        layer = Layer(het, w, q, k, v, u, rho)
        res = time_layer(layer, steps, warmup)
        eff = W.effective_flops(w, [W.dense_count(w.n_tokens, rho)] * w.batch)
        ms = res["step_ms_median"]
        row = {"workload": name, "rho": rho, "window": list(w.window), "batch": w.batch, "heads": w.heads,
               "tokens": w.n_tokens, "ms_per_layer": round(ms, 5), "route_ms": round(res["route_ms_median"], 5),
               "local_ms": round(res["local_ms_median"], 5), "dense_ms": round(res["dense_ms_median"], 5),
               "effective_TFLOPs": round(eff / (ms * 1e-3) / 1e12, 2),
               "pct_mfma_peak": round(100.0 * eff / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        log(f"[bench] sweep {row}")
        rows.append(row)
        del layer
    cache.clear()
    torch.cuda.synchronize()
    return rows


def run_oracle_full(W, everything: bool = False):
    """The fp64 oracle on whole layers (route + every dense and local row),
    timed on the host cores: the tiny case and the Wan-1.3B layer at rho =
    0.2 (about a minute on 16 threads), or with `everything` also the rho
    sweep and the other workloads (tens of minutes)."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    cases = [("tiny", None), ("wan13b", None)]
    if everything:
        cases += [("wan13b", r) for r in W.RHO_SWEEP if r != 0.2] + [("wan5b", None), ("long", None)]
    rows = []
    for name, r in cases:
        w = W.WORKLOADS[name]
        rho = w.rho if r is None else r
        qn, kn, vn = W.make_qkv(w)
        un = W.make_u(w)
        t0 = time.perf_counter()
        rt = oracle.route_top_rho(un, rho)
        t1 = time.perf_counter()
        all_rows = np.arange(w.batch * w.n_tokens, dtype=np.int64)
        oracle.attend_rows(qn, kn, vn, w.grid, w.window, w.softmax_scale, rt.mask, all_rows, nthreads=threads)
        t2 = time.perf_counter()
        eff = W.effective_flops(w.with_(rho=rho))
        row = {"workload": name, "rho": rho, "route_s": round(t1 - t0, 3), "forward_s": round(t2 - t1, 2),
               "effective_TFLOPs": round(eff / (t2 - t0) / 1e12, 5), "threads": threads, "cpu": cpu_model()}
        log(f"[bench] oracle {row}")
        rows.append(row)
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan13b",
                    choices=["wan13b", "wan5b", "long", "tiny", "wan13b_w11", "wan5b_w11"])
    ap.add_argument("--window", default=None, help="override the workload's window, e.g. 11,11,11")
    ap.add_argument("--rho", type=float, default=None, help="override the workload's rho")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-baseline", action="store_true")
    ap.add_argument("--cpu-stride", type=int, default=4)
    ap.add_argument("--lib", default=None, help="load this libhetattn.so instead of the in-tree one")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (calibrates HBM counters)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the rho sweep, the window ablation and the other workloads")
    ap.add_argument("--router", default="top_rho", choices=["top_rho", "uniform", "random"],
                    help="routing of the timed layer (the ablation routers of the routing study)")
    ap.add_argument("--border", default="shift", choices=["shift", "cut"],
                    help="local window border: shifted inside the grid, or cut at it")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing het_attn_backward (dQ, dK, dV) on the same layer")
    ap.add_argument("--swap-ratio", type=float, default=0.07,
                    help="ratio r of the per-block random swap timed beside the step (0 skips it)")
    ap.add_argument("--oracle-full", action="store_true",
                    help="also time the fp64 oracle on the whole tiny and Wan-1.3B layers (about a minute)")
    ap.add_argument("--oracle-full-all", action="store_true",
                    help="with --oracle-full: also the rho sweep and the other workloads (tens of minutes)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the layer shards by (sample, head) with no collectives between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB x 5")
        return

    import uncertainty_routed_heterogeneous_amd as het
    import workloads as W

    if args.lib:
        het.load_library(os.path.abspath(args.lib))
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = W.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        w = w.with_(dtype="bf16")
    rho = w.rho if args.rho is None else args.rho
    if args.window:
        w = w.with_(window=tuple(int(x) for x in args.window.split(",")))
    log(f"[bench] workload={w.name} grid={w.grid} B={w.batch} heads={w.heads} D={w.head_dim} "
        f"rho={rho} window={w.window}")
    qn, kn, vn = W.make_qkv(w)
    un = W.make_u(w)
    to_bf16 = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    q, k, v = to_bf16(qn), to_bf16(kn), to_bf16(vn)
    u = torch.from_numpy(un).cuda()
    torch.cuda.synchronize()

    layer = Layer(het, w, q, k, v, u, rho, router=args.router, border=args.border)
    res = time_layer(layer, args.steps, args.warmup)
    n_dense = [W.dense_count(w.n_tokens, rho)] * w.batch
    eff_flop = effective_flops_routed(w, layer.mask.cpu().numpy(), args.border)
    dense_flop = 4.0 * w.head_dim * w.heads * sum(kd * w.n_tokens for kd in n_dense)
    bytes_el = 2
    BNHD = w.batch * w.n_tokens * w.heads * w.head_dim
    n_local = sum(w.n_tokens - kd for kd in n_dense)
    local_bytes = 2 * BNHD * bytes_el + 2 * n_local * w.heads * w.head_dim * bytes_el
    route_bytes = 13 * w.batch * w.n_tokens
    value = eff_flop / (res["ms_per_step"] * 1e-3) / 1e12
    dense_tflops = dense_flop / (res["dense_ms"] * 1e-3) / 1e12
    traffic = read_traffic(dense_flop / (4.0 * w.head_dim))
    log(f"[bench] ms/step={res['ms_per_step']:.4f} route={res['route_ms']:.4f} "
        f"local={res['local_ms']:.4f} dense={res['dense_ms']:.4f} -> {value:.1f} TFLOP/s effective, "
        f"dense kernel {dense_tflops:.1f} TFLOP/s")

    cold = None
    if not args.no_cold:
        # 512 MiB write between steps evicts L2 (4 MiB per XCD) and the 256 MiB last-level cache.
        scrub = torch.empty(512 * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        rc = time_layer(layer, max(10, args.steps // 2), 2, scrub=scrub)
        del scrub
        cold = {"scrub_MiB": 512, "steps": max(10, args.steps // 2), "ms_per_step_median": round(rc["step_ms_median"], 5),
                "route_ms_median": round(rc["route_ms_median"], 5), "local_ms_median": round(rc["local_ms_median"], 5),
                "dense_ms_median": round(rc["dense_ms_median"], 5)}
        log(f"[bench] cold: {cold}")

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: HetA attention layer, B={w.batch}, {w.heads} heads, "
                               f"head_dim {w.head_dim}, grid {w.grid[0]}x{w.grid[1]}x{w.grid[2]}",
                   "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim, "grid": list(w.grid),
                   "tokens": w.n_tokens, "rho": rho, "dense_tokens": n_dense,
                   "window": list(w.window), "u": w.u_kind, "effective_flop": eff_flop,
                   "router": args.router, "border": args.border},
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma",
                     "kernel": "dense call: dense_bf16_kernel<128,false> + dense_merge_kernel<128,false>",
                     "achieved": round(dense_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dense_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "avg_launch_ms": round(res["dense_ms"], 5),
                     "flop_per_launch": dense_flop},
        "kernels": {
            "route_ms": round(res["route_ms"], 5),
            "route_GBps": round(route_bytes / (res["route_ms"] * 1e-3) / 1e9, 1),
            "local_ms": round(res["local_ms"], 5),
            "local_GBps": round(local_bytes / (res["local_ms"] * 1e-3) / 1e9, 1),
            "local_frac_hbm": round(local_bytes / (res["local_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "dense_ms": round(res["dense_ms"], 5),
            "route_ms_median": round(res["route_ms_median"], 5),
            "local_ms_median": round(res["local_ms_median"], 5),
            "dense_ms_median": round(res["dense_ms_median"], 5),
            "ms_per_step_median": round(res["step_ms_median"], 5),
            # the route is computed once per denoising step and shared by every block
            "ms_per_layer_route_amortized_30": round(res["route_ms_median"] / 30 + res["local_ms_median"] +
                                                     res["dense_ms_median"], 5),
        },
    }
    if cold is not None:
        out["cold"] = cold

    if not args.no_backward:
        bms = time_backward(layer, max(5, args.steps // 5))
        bms_re = time_backward(layer, max(5, args.steps // 5), with_lse=False)
        bflop = 2.5 * eff_flop  # five products (S, dP, dV, dQ, dK) against the forward's two
        out["backward"] = {"ms_median": round(bms, 4), "lse": "from het_attn_forward_lse",
                           "ms_median_lse_recomputed": round(bms_re, 4), "algorithmic_flop": bflop,
                           "TFLOPs": round(bflop / (bms * 1e-3) / 1e12, 2),
                           "frac_bf16_peak": round(bflop / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] backward: {out['backward']}")

    if args.swap_ratio > 0:
        # Per-block random swap: one launch makes the routes of all 30 blocks
        # of a Wan step; it depends only on the step's route.
        s30 = time_swap(layer, args.swap_ratio, 30, max(10, args.steps // 2))
        s1 = time_swap(layer, args.swap_ratio, 1, max(10, args.steps // 2))
        out["swap"] = {"ratio": args.swap_ratio, "blocks": 30, "ms_30_blocks_median": round(s30, 5),
                       "ms_1_block_median": round(s1, 5), "ms_per_block_amortized": round(s30 / 30, 5),
                       "GBps_30_blocks": round(30 * 10 * w.batch * w.n_tokens / (s30 * 1e-3) / 1e9, 1)}
        log(f"[bench] swap: {out['swap']}")

    if not args.no_dense_baseline and rho < 1.0:
        dl = Layer(het, w, q, k, v, u, 1.0)
        rd = time_layer(dl, max(5, args.steps // 5), max(2, args.warmup // 5))
        out["dense_rho1"] = {"ms_per_step": round(rd["ms_per_step"], 5),
                             "dense_kernel_TFLOPs": round(4.0 * w.head_dim * w.heads * w.batch *
                                                          w.n_tokens ** 2 / (rd["dense_ms"] * 1e-3) / 1e12, 2),
                             "speedup_vs_rho1": round(rd["ms_per_step"] / res["ms_per_step"], 3)}
        log(f"[bench] rho=1 dense path: {rd['ms_per_step']:.4f} ms/step "
            f"({out['dense_rho1']['speedup_vs_rho1']}x slower than rho={rho})")
        del dl

    if not args.no_sweep and args.workload == "wan13b" and args.window is None and args.rho is None:
        out["sweep"] = run_sweep(het, W, torch, (q, k, v, u), max(10, args.steps // 5), 3)

    if args.oracle_full:
        out["oracle_full"] = run_oracle_full(W, args.oracle_full_all)

    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 CPU oracle on a sample ...")
        out["cpu_baseline"] = cpu_baseline(w, qn, kn, vn, un, rho, args.cpu_stride)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
