"""Uncertainty-routed heterogeneous attention on AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libhetattn.so`` (C ABI in ``include/hetattn.h``).
This module only marshals arguments: every step of the layer runs in the HIP
kernels of ``csrc/``.  PyTorch supplies device memory and the current stream.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT, arXiv 2609.31050).

    r = route(u, grid, window, q.shape, rho=0.2)   # §3.2.2 Eqs. 11-12
    rb = swap(r, 0.07, seed, step, n_blocks=30)    # §3.2.2, per-block swap
    o = forward(q, k, v, rb[block])                # §3.2.2 Eq. 13

The library is loaded on first use; if it is missing the call raises -- there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhetattn.so")

HET_OK, HET_ERR_INVALID_ARG, HET_ERR_UNSUPPORTED, HET_ERR_WORKSPACE, HET_ERR_HIP = range(5)
HET_BF16, HET_F32 = 0, 1
HET_TOP_RHO, HET_MEAN_STD, HET_UNIFORM = 0, 1, 2
HET_BORDER_SHIFT, HET_BORDER_CUT = 0, 1
ABI_VERSION = 5
_BORDERS = {"shift": HET_BORDER_SHIFT, "cut": HET_BORDER_CUT}


class HetAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("win_t", ctypes.c_int32), ("win_h", ctypes.c_int32), ("win_w", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("border", ctypes.c_int32)]


class RouteStruct(ctypes.Structure):
    _fields_ = [("mask", ctypes.c_void_p), ("dense_idx", ctypes.c_void_p),
                ("local_idx", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("thresh", ctypes.c_void_p), ("dense_count_host", ctypes.c_int32)]


# Exported symbols and their ctypes signatures (the names of include/hetattn.h).
SIGNATURES = {
    "het_attn_abi_version": (ctypes.c_int, []),
    "het_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "het_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "het_attn_route_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "het_attn_route": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_double, ctypes.POINTER(RouteStruct), ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]),
}
SIGNATURES["het_attn_backward_workspace_bytes"] = (ctypes.c_size_t, [ctypes.POINTER(Shape)])
SIGNATURES["het_attn_backward"] = (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.POINTER(RouteStruct),
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_size_t, ctypes.c_void_p])
SIGNATURES["het_attn_route_random"] = (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_double, ctypes.c_uint64,
                                                      ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int32,
                                                      ctypes.POINTER(RouteStruct), ctypes.c_void_p])
SIGNATURES["het_attn_swap"] = (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(RouteStruct),
                                              ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
                                              ctypes.c_uint32, ctypes.c_int32,
                                              ctypes.POINTER(RouteStruct), ctypes.c_void_p])
_ATTN_ARGS = [ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
              ctypes.POINTER(RouteStruct), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
              ctypes.c_void_p]
for _name in ("het_attn_forward", "het_attn_dense", "het_attn_local"):
    SIGNATURES[_name] = (ctypes.c_int, _ATTN_ARGS)
SIGNATURES["het_attn_forward_noalloc"] = (ctypes.c_int, _ATTN_ARGS[:6] + [ctypes.c_void_p])
SIGNATURES["het_attn_forward_lse"] = (ctypes.c_int, _ATTN_ARGS[:6] + [ctypes.c_void_p] + _ATTN_ARGS[6:])
SIGNATURES["het_attn_backward_lse"] = (ctypes.c_int, SIGNATURES["het_attn_backward"][1][:7] + [ctypes.c_void_p]
                                       + SIGNATURES["het_attn_backward"][1][7:])

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libhetattn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m uncertainty_routed_heterogeneous_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.het_attn_abi_version() != ABI_VERSION:
            raise RuntimeError("libhetattn.so ABI version mismatch")
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().het_status_string(int(status)).decode()


def make_shape(batch, heads, head_dim, grid, window, dtype, scale=0.0, border="shift") -> Shape:
    return Shape(int(batch), int(heads), int(head_dim), *[int(g) for g in grid],
                 *[int(w) for w in window], int(dtype), float(scale), _BORDERS[border])


def _stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _on_stream(stream):
    """Context for the allocations of a call that runs on `stream`: tensors
    allocated inside belong to that stream in PyTorch's caching allocator, so
    a workspace freed when the call returns is not handed to other work while
    the call's kernels still use it."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check_out(t, like, what: str) -> None:
    if (tuple(t.shape) != tuple(like.shape) or t.dtype != like.dtype or t.device != like.device
            or not t.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous tensor of q's shape, dtype and device")


def _check_attn(q, k, v, r: "Route", tensors=()) -> None:
    """Shape checks of an attention call, before anything touches a device:
    the kernels size every index from the route's grid and read the route's
    [B, N] buffers, so q must hold B samples of prod(grid) tokens."""
    for t in (q, k, v) + tuple(tensors):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k, v (and o, dout) must be contiguous [B, N, heads, D] tensors")
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    for t in tensors:
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("o and dout must have q's shape and dtype")
    B, N = int(q.shape[0]), int(q.shape[1])
    if math.prod(r.grid) != N:
        raise ValueError(f"q holds {N} tokens per sample but the route's grid {tuple(r.grid)} "
                         f"holds {math.prod(r.grid)}")
    for name in ("mask", "dense_idx", "local_idx"):
        if tuple(getattr(r, name).shape) != (B, N):
            raise ValueError(f"route.{name} is {tuple(getattr(r, name).shape)}, not [B, N] = {(B, N)}")
    if tuple(r.counts.shape) != (B, 2):
        raise ValueError("route.counts must be [B, 2]")
    for t in (q, k, v) + tuple(tensors):
        if not t.is_cuda:
            raise ValueError("q, k, v (and o, dout) must be CUDA tensors")
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    for name in ("mask", "dense_idx", "local_idx", "counts"):
        if getattr(r, name).device != q.device:
            raise ValueError(f"route.{name} is not on q's device")


@dataclass
class Route:
    """Result of :func:`route`: device tensors plus the host-side dense count."""
    mask: "object"        # uint8 [B, N], 1 = local
    dense_idx: "object"   # int32 [B, N]
    local_idx: "object"   # int32 [B, N]
    counts: "object"      # int32 [B, 2]
    thresh: "object"      # float64 [B]
    dense_count_host: int
    grid: tuple
    window: tuple

    def as_struct(self) -> RouteStruct:
        return RouteStruct(self.mask.data_ptr(), self.dense_idx.data_ptr(), self.local_idx.data_ptr(),
                           self.counts.data_ptr(), self.thresh.data_ptr(), int(self.dense_count_host))


def _dtype_code(t) -> int:
    import torch
    if t == torch.bfloat16:
        return HET_BF16
    if t == torch.float32:
        return HET_F32
    raise TypeError(f"unsupported dtype {t}")


def route(u, grid, window, heads: int, head_dim: int, dtype, rho: float | None = None,
          c: float | None = None, stream=None) -> Route:
    """Threshold, mask and compaction for u [B, N] (float32, on the GPU)."""
    import torch
    if (rho is None) == (c is None):
        raise ValueError("give exactly one of rho (top-rho) or c (mean-std)")
    if u.dtype != torch.float32 or u.dim() != 2 or not u.is_cuda or not u.is_contiguous():
        raise ValueError("u must be a contiguous float32 [B, N] CUDA tensor")
    B, N = u.shape
    if math.prod(grid) != N:
        raise ValueError("grid does not match N")
    dev = u.device
    with _on_stream(stream):
        r = Route(torch.empty((B, N), dtype=torch.uint8, device=dev),
                  torch.empty((B, N), dtype=torch.int32, device=dev),
                  torch.empty((B, N), dtype=torch.int32, device=dev),
                  torch.empty((B, 2), dtype=torch.int32, device=dev),
                  torch.empty((B,), dtype=torch.float64, device=dev), -1, tuple(grid), tuple(window))
    shape = make_shape(B, heads, head_dim, grid, window, _dtype_code(dtype))
    rs = r.as_struct()
    mode, param = (HET_TOP_RHO, rho) if rho is not None else (HET_MEAN_STD, c)
    lib = load_library()
    ws_bytes = int(lib.het_attn_route_workspace_bytes(ctypes.byref(shape))) if mode == HET_TOP_RHO else 0
    ws = None
    if ws_bytes:
        # Stream-ordered scratch: freed after the launch, reused only by work
        # that the caching allocator orders after it on the same stream.
        with _on_stream(stream):
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.het_attn_route(ctypes.byref(shape), u.data_ptr(), mode, float(param), ctypes.byref(rs),
                            ws.data_ptr() if ws is not None else None, ws_bytes, _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, "het_attn_route")
    r.dense_count_host = rs.dense_count_host
    return r


def _new_routes(n_blocks: int, B: int, N: int, device):
    import torch
    return (torch.empty((n_blocks, B, N), dtype=torch.uint8, device=device),
            torch.empty((n_blocks, B, N), dtype=torch.int32, device=device),
            torch.empty((n_blocks, B, N), dtype=torch.int32, device=device),
            torch.empty((n_blocks, B, 2), dtype=torch.int32, device=device),
            torch.empty((n_blocks, B), dtype=torch.float64, device=device))


def route_uniform(batch: int, grid, window, rho: float, device=None, stream=None) -> Route:
    """Fixed uniform routing (HET_UNIFORM): the lattice floor(j*N/K), j < K."""
    import torch
    N = math.prod(grid)
    with _on_stream(stream):
        bufs = [b[0] for b in _new_routes(1, batch, N, device or torch.device("cuda"))]
    r = Route(*bufs, -1, tuple(grid), tuple(window))
    shape = make_shape(batch, 1, 64, grid, window, HET_F32)
    rs = r.as_struct()
    st = load_library().het_attn_route(ctypes.byref(shape), None, HET_UNIFORM, float(rho),
                                       ctypes.byref(rs), None, 0, _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, "het_attn_route")
    r.dense_count_host = rs.dense_count_host
    return r


def route_random(batch: int, grid, window, rho: float, seed: int, step: int, block: int = 0,
                 n_blocks: int = 1, device=None, stream=None):
    """Random routing per block (het_attn_route_random): a list of n_blocks
    Route objects viewing one allocation, route l for block `block + l`."""
    import torch
    N = math.prod(grid)
    with _on_stream(stream):
        bufs = _new_routes(int(n_blocks), batch, N, device or torch.device("cuda"))
    rs = RouteStruct(*[b.data_ptr() for b in bufs], -1)
    shape = make_shape(batch, 1, 64, grid, window, HET_F32)
    st = load_library().het_attn_route_random(ctypes.byref(shape), float(rho), int(seed) & (2**64 - 1),
                                              int(step) & 0xffffffff, int(block) & 0xffffffff,
                                              int(n_blocks), ctypes.byref(rs), _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, "het_attn_route_random")
    return [Route(*[b[l] for b in bufs], rs.dense_count_host, tuple(grid), tuple(window))
            for l in range(int(n_blocks))]


def swap(r: Route, ratio: float, seed: int, step: int, block: int = 0, n_blocks: int = 1,
         in_place: bool = False, stream=None):
    """Per-block random swap of a route (het_attn_swap).

    Returns the routes of blocks block .. block + n_blocks - 1 as a list of
    Route objects viewing one allocation ([n_blocks, B, N] tensors); with
    in_place=True (n_blocks = 1 only) `r` itself is rewritten and returned."""
    import torch
    B, N = r.mask.shape
    dev = r.mask.device
    if in_place:
        if n_blocks != 1:
            raise ValueError("in_place needs n_blocks == 1")
        outs = [r]
        rs_out = r.as_struct()
    else:
        nb = int(n_blocks)
        with _on_stream(stream):
            mask, di, li, cnt, th = _new_routes(nb, B, N, dev)
        outs = [Route(mask[l], di[l], li[l], cnt[l], th[l], r.dense_count_host, r.grid, r.window)
                for l in range(nb)]
        rs_out = RouteStruct(mask.data_ptr(), di.data_ptr(), li.data_ptr(), cnt.data_ptr(),
                             th.data_ptr(), -1)
    shape = make_shape(B, 1, 64, r.grid, r.window, HET_F32)
    rs_in = r.as_struct()
    st = load_library().het_attn_swap(ctypes.byref(shape), ctypes.byref(rs_in), float(ratio),
                                      int(seed) & (2**64 - 1), int(step) & 0xffffffff,
                                      int(block) & 0xffffffff, int(n_blocks), ctypes.byref(rs_out),
                                      _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, "het_attn_swap")
    for o in outs:
        o.dense_count_host = rs_out.dense_count_host
    return outs


def workspace_bytes(shape: Shape) -> int:
    return int(load_library().het_attn_workspace_bytes(ctypes.byref(shape)))


def forward(q, k, v, r: Route, scale: float | None = None, out=None, stream=None,
            part: str = "both", border: str = "shift", return_lse: bool = False):
    """Heterogeneous attention for contiguous [B, N, heads, D] CUDA tensors.

    part = "both" (het_attn_forward), "dense" (het_attn_dense: rows with
    m_i = 0 only) or "local" (het_attn_local: rows with m_i = 1 only).
    border = "shift" (window shifted inside the grid) or "cut" (cut at it).
    return_lse (part "both", bf16): also return the rows' log-sum-exp,
    [B, heads, N] fp32 in log2 units (het_attn_forward_lse), for backward()."""
    import torch
    _check_attn(q, k, v, r)
    if out is not None:
        _check_out(out, q, "out")
    if return_lse and part != "both":
        raise ValueError("return_lse needs part='both'")
    B, N, H, D = q.shape
    shape = make_shape(B, H, D, r.grid, r.window, _dtype_code(q.dtype), scale or 0.0, border)
    ws_n = workspace_bytes(shape)
    with _on_stream(stream):
        if out is None:
            out = torch.empty_like(q)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device) if ws_n else None
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    rs = r.as_struct()
    if return_lse:
        st = load_library().het_attn_forward_lse(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 ctypes.byref(rs), out.data_ptr(), lse.data_ptr(),
                                                 ws.data_ptr() if ws is not None else None, ws_n,
                                                 _stream_handle(stream))
        if st != HET_OK:
            raise HetAttnError(st, "het_attn_forward_lse")
        return out, lse
    name = {"both": "het_attn_forward", "dense": "het_attn_dense", "local": "het_attn_local"}[part]
    st = getattr(load_library(), name)(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       ctypes.byref(rs), out.data_ptr(),
                                       ws.data_ptr() if ws is not None else None, ws_n,
                                       _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, name)
    return out


def forward_noalloc(q, k, v, r: Route, out, scale: float | None = None, stream=None, border: str = "shift"):
    """het_attn_forward_noalloc: het_attn_forward into the caller's `out`
    with the library's static scratch, so that neither this call nor the
    library allocates device memory.  Calls that overlap in time on one
    device share that scratch and must be ordered by the caller."""
    _check_attn(q, k, v, r)
    _check_out(out, q, "out")
    B, N, H, D = q.shape
    shape = make_shape(B, H, D, r.grid, r.window, _dtype_code(q.dtype), scale or 0.0, border)
    rs = r.as_struct()
    st = load_library().het_attn_forward_noalloc(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 ctypes.byref(rs), out.data_ptr(), _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, "het_attn_forward_noalloc")
    return out


def backward(q, k, v, r: Route, o, dout, scale: float | None = None, stream=None, border: str = "shift",
             lse=None, out=None):
    """(dQ, dK, dV) of forward(q, k, v, r) = o for dL/dO = dout (het_attn_backward).

    lse: the rows' log-sum-exp from forward(..., return_lse=True) for the same
    inputs (het_attn_backward_lse: not computed again).
    out: optional (dq, dk, dv) tensors of q's shape, dtype and device to write."""
    import torch
    _check_attn(q, k, v, r, (o, dout))
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be (dq, dk, dv)")
        for t, name in zip(out, ("dq", "dk", "dv")):
            _check_out(t, q, name)
    B, N, H, D = q.shape
    shape = make_shape(B, H, D, r.grid, r.window, _dtype_code(q.dtype), scale or 0.0, border)
    lib = load_library()
    ws_n = int(lib.het_attn_backward_workspace_bytes(ctypes.byref(shape)))
    with _on_stream(stream):
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
        dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    rs = r.as_struct()
    if lse is not None:
        if (not lse.is_cuda or lse.device != q.device or lse.dtype != torch.float32 or not lse.is_contiguous()
                or tuple(lse.shape) != (B, H, N)):
            raise ValueError("lse must be a contiguous [B, heads, N] float32 CUDA tensor")
        st = lib.het_attn_backward_lse(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       ctypes.byref(rs), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws_n,
                                       _stream_handle(stream))
        if st != HET_OK:
            raise HetAttnError(st, "het_attn_backward_lse")
        return dq, dk, dv
    st = lib.het_attn_backward(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(rs),
                               o.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                               ws.data_ptr(), ws_n, _stream_handle(stream))
    if st != HET_OK:
        raise HetAttnError(st, "het_attn_backward")
    return dq, dk, dv
