"""Plain fp64 CPU oracle for uncertainty-routed heterogeneous attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import
this package.  It shares no code with the HIP path and the HIP path never
calls it.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT, arXiv 2609.31050), full text.

The arithmetic lives in ``hetattn_oracle.c`` (double precision, plain loops);
this module only marshals numpy arrays through ctypes.  Functions:

* :func:`route_top_rho`  -- dense set = the round(rho*N) largest u, ties by
  token index (quantile reading of [HetA §3.2.2 Eqs. 11-12]).
* :func:`route_mean_std` -- T = mu + c*sigma, m_i = 1[u_i < T]
  ([HetA §3.2.2 Eqs. 11-12]).
* :func:`attend_rows`    -- Eq. 13 for chosen rows: dense rows use Eq. 2 over
  all N keys, local rows use Eq. 3 over the 3D window ([HetA §3.1.1]).
* :func:`forward`        -- :func:`attend_rows` over every token.
* :func:`attention_weights` -- the softmax weights of one (row, head).
* :func:`row_lse`        -- log of the softmax normaliser of chosen rows, the
  statistic the gradient of the layer reuses.
* :func:`backward`, :func:`backward_dq_rows`, :func:`backward_kv_rows` -- the
  gradients of the layer with the route held fixed: all of dQ, dK, dV; dQ of
  chosen rows; dK and dV of chosen keys and heads.

Parity pins for every function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hetattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Tests that plant mistakes in a copy of the oracle point this at the copy.
_LIB_OVERRIDE = os.environ.get("HETATTN_ORACLE_LIB")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"  # several test workers may build at once
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_route_top_rho.argtypes = [P, i, i, ctypes.c_double, P, P, P, P, P]
        lib.oracle_route_mean_std.argtypes = [P, i, i, ctypes.c_double, P, P, P, P, P]
        lib.oracle_window_axis.argtypes = [i, i, i, P, P]
        lib.oracle_window_axis_cut.argtypes = [i, i, i, P, P]
        lib.oracle_attend_rows.argtypes = [P, P, P, i, i, i, i, i, i, i, i, i, i,
                                           ctypes.c_double, P, P, ctypes.c_long, P, i]
        lib.oracle_attention_weights.argtypes = [P, P, i, i, i, i, i, i, i, i, i, i,
                                                 ctypes.c_double, P, ctypes.c_long, i, P]
        lib.oracle_row_lse.argtypes = [P, P, i, i, i, i, i, i, i, i, i, i,
                                       ctypes.c_double, P, P, ctypes.c_long, P, i]
        lib.oracle_route_uniform.argtypes = [i, i, ctypes.c_double, P, P, P, P]
        lib.oracle_attend_backward.argtypes = [P, P, P, P, i, i, i, i, i, i, i, i, i, i,
                                               ctypes.c_double, P, P, P, P, i]
        lib.oracle_attend_backward_dq_rows.argtypes = [P, P, P, P, i, i, i, i, i, i, i, i, i, i,
                                                       ctypes.c_double, P, P, ctypes.c_long, P, i]
        lib.oracle_attend_backward_kv_rows.argtypes = [P, P, P, P, i, i, i, i, i, i, i, i, i, i,
                                                       ctypes.c_double, P, P, ctypes.c_long, P, i, P, P, i]
        lib.oracle_route_random.argtypes = [i, i, ctypes.c_double, ctypes.c_ulonglong, ctypes.c_uint,
                                            ctypes.c_uint, P, P, P, P]
        lib.oracle_philox4x32_10.argtypes = [P, P, P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_swap_draws.argtypes = [i, ctypes.c_uint, ctypes.c_ulonglong, ctypes.c_uint,
                                          ctypes.c_uint, P]
        lib.oracle_swap_draws.restype = None
        lib.oracle_route_swap.argtypes = [P, i, i, ctypes.c_double, ctypes.c_ulonglong, ctypes.c_uint,
                                          ctypes.c_uint, P, P, P, P]
        for fn in (lib.oracle_route_top_rho, lib.oracle_route_mean_std, lib.oracle_window_axis,
                   lib.oracle_attend_rows, lib.oracle_attention_weights, lib.oracle_route_swap,
                   lib.oracle_window_axis_cut, lib.oracle_route_uniform, lib.oracle_route_random,
                   lib.oracle_attend_backward, lib.oracle_attend_backward_dq_rows, lib.oracle_row_lse,
                   lib.oracle_attend_backward_kv_rows):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


@dataclass
class Route:
    mask: np.ndarray       # uint8 [B, N], 1 = local
    dense_idx: np.ndarray  # int32 [B, N], ascending, -1 past the count
    local_idx: np.ndarray  # int32 [B, N], ascending, -1 past the count
    counts: np.ndarray     # int32 [B, 2] = (dense, local)
    thresh: np.ndarray     # float64 [B]


def _route(fn_name: str, u: np.ndarray, param: float) -> Route:
    u = np.ascontiguousarray(u, dtype=np.float32)
    if u.ndim != 2:
        raise ValueError("u must be [B, N]")
    B, N = u.shape
    mask = np.empty((B, N), np.uint8)
    di = np.empty((B, N), np.int32)
    li = np.empty((B, N), np.int32)
    counts = np.empty((B, 2), np.int32)
    thresh = np.empty(B, np.float64)
    rc = getattr(_load(), fn_name)(_ptr(u), B, N, float(param), _ptr(mask), _ptr(di),
                                   _ptr(li), _ptr(counts), _ptr(thresh))
    if rc != 0:
        raise ValueError(f"{fn_name} rejected its arguments (rc={rc})")
    return Route(mask, di, li, counts, thresh)


def route_top_rho(u: np.ndarray, rho: float) -> Route:
    return _route("oracle_route_top_rho", u, rho)


def route_mean_std(u: np.ndarray, c: float) -> Route:
    return _route("oracle_route_mean_std", u, c)


def philox4x32_10(ctr, key) -> tuple:
    """Philox4x32-10 (Salmon et al., SC'11) of a 4-word counter and a 2-word key."""
    c = np.array(ctr, dtype=np.uint32)
    kk = np.array(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(kk), _ptr(out))
    return tuple(int(x) for x in out)


def route_swap(mask_in: np.ndarray, r: float, seed: int, step: int, block: int) -> Route:
    """Per-block random swap of a route ([HetA §3.2.2 after Eq. 12; App. B,
    Table 8]); see oracle_route_swap.  thresh is not defined by the swap and
    is returned as NaN."""
    m = np.ascontiguousarray(mask_in, dtype=np.uint8)
    if m.ndim != 2:
        raise ValueError("mask must be [B, N]")
    B, N = m.shape
    mask = np.empty((B, N), np.uint8)
    di = np.empty((B, N), np.int32)
    li = np.empty((B, N), np.int32)
    counts = np.empty((B, 2), np.int32)
    rc = _load().oracle_route_swap(_ptr(m), B, N, float(r), int(seed), int(step), int(block),
                                   _ptr(mask), _ptr(di), _ptr(li), _ptr(counts))
    if rc != 0:
        raise ValueError(f"oracle_route_swap rejected its arguments (rc={rc})")
    return Route(mask, di, li, counts, np.full(B, np.nan))


def swap_draws(N: int, b: int, seed: int, step: int, block: int) -> np.ndarray:
    """The per-token draws route_swap ranks, for sample b: uint32 [N]."""
    out = np.empty(N, np.uint32)
    _load().oracle_swap_draws(int(N), int(b), int(seed), int(step), int(block), _ptr(out))
    return out


def _routes_out(B: int, N: int):
    return (np.empty((B, N), np.uint8), np.empty((B, N), np.int32), np.empty((B, N), np.int32),
            np.empty((B, 2), np.int32))


def route_uniform(B: int, N: int, rho: float) -> Route:
    """Fixed uniform routing ([HetA §5.1, Table 6]; see oracle_route_uniform).
    thresh is not defined and is returned as NaN."""
    mask, di, li, counts = _routes_out(B, N)
    rc = _load().oracle_route_uniform(int(B), int(N), float(rho), _ptr(mask), _ptr(di), _ptr(li),
                                      _ptr(counts))
    if rc != 0:
        raise ValueError(f"oracle_route_uniform rejected its arguments (rc={rc})")
    return Route(mask, di, li, counts, np.full(B, np.nan))


def route_random(B: int, N: int, rho: float, seed: int, step: int, block: int) -> Route:
    """Random routing per block ([HetA §5.1, Table 6]; see oracle_route_random).
    thresh is not defined and is returned as NaN."""
    mask, di, li, counts = _routes_out(B, N)
    rc = _load().oracle_route_random(int(B), int(N), float(rho), int(seed), int(step), int(block),
                                     _ptr(mask), _ptr(di), _ptr(li), _ptr(counts))
    if rc != 0:
        raise ValueError(f"oracle_route_random rejected its arguments (rc={rc})")
    return Route(mask, di, li, counts, np.full(B, np.nan))


_BORDER = {"shift": 0, "cut": 1, "truncate": 1}  # "truncate" = "cut"


def window_axis(S: int, k: int, pos: int, border: str = "shift") -> tuple[int, int]:
    start = ctypes.c_int()
    length = ctypes.c_int()
    fn = _load().oracle_window_axis if _BORDER[border] == 0 else _load().oracle_window_axis_cut
    rc = fn(S, k, pos, ctypes.addressof(start), ctypes.addressof(length))
    if rc != 0:
        raise ValueError("bad window arguments")
    return start.value, length.value


def _as_f32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def attend_rows(q, k, v, grid, window, scale, mask, rows, nthreads: int = 0,
                border: str = "shift") -> np.ndarray:
    """Outputs [len(rows), heads, D] (float64) for rows = b*N + n."""
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    B, N, H, D = q.shape
    T, Hg, Wg = grid
    if T * Hg * Wg != N or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("shape mismatch")
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), np.float64)
    wt, wh, ww = window
    rc = _load().oracle_attend_rows(_ptr(q), _ptr(k), _ptr(v), B, H, D, T, Hg, Wg, wt, wh, ww,
                                    _BORDER[border], float(scale), _ptr(mask), _ptr(rows), rows.size, _ptr(out),
                                    int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attend_rows rejected its arguments (rc={rc})")
    return out


def forward(q, k, v, grid, window, scale, mask, nthreads: int = 0,
            border: str = "shift") -> np.ndarray:
    """Outputs [B, N, heads, D] (float64) for every token."""
    B, N, H, D = q.shape
    rows = np.arange(B * N, dtype=np.int64)
    return attend_rows(q, k, v, grid, window, scale, mask, rows, nthreads,
                       border).reshape(B, N, H, D)


def row_lse(q, k, grid, window, scale, mask, rows, nthreads: int = 0, border: str = "shift") -> np.ndarray:
    """[len(rows), heads] (float64): log sum_j exp(scale * q.k_j) over each
    row's key set, natural log, for rows = b*N + n."""
    q, k = _as_f32(q), _as_f32(k)
    B, N, H, D = q.shape
    T, Hg, Wg = grid
    if T * Hg * Wg != N or k.shape != q.shape:
        raise ValueError("shape mismatch")
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H), np.float64)
    wt, wh, ww = window
    rc = _load().oracle_row_lse(_ptr(q), _ptr(k), B, H, D, T, Hg, Wg, wt, wh, ww, _BORDER[border],
                                float(scale), _ptr(mask), _ptr(rows), rows.size, _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_row_lse rejected its arguments (rc={rc})")
    return out


def attention_weights(q, k, grid, window, scale, mask, row: int, head: int,
                      border: str = "shift") -> np.ndarray:
    q, k = _as_f32(q), _as_f32(k)
    B, N, H, D = q.shape
    T, Hg, Wg = grid
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    w = np.empty(N, np.float64)
    wt, wh, ww = window
    rc = _load().oracle_attention_weights(_ptr(q), _ptr(k), B, H, D, T, Hg, Wg, wt, wh, ww,
                                          _BORDER[border], float(scale), _ptr(mask), int(row), int(head), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_attention_weights rejected its arguments")
    return w


def backward(q, k, v, dout, grid, window, scale, mask, nthreads: int = 0, border: str = "shift"):
    """(dQ, dK, dV) as float64 [B, N, heads, D] arrays (oracle_attend_backward)."""
    q, k, v, dout = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, N, H, D = q.shape
    T, Hg, Wg = grid
    if T * Hg * Wg != N or any(x.shape != q.shape for x in (k, v, dout)):
        raise ValueError("shape mismatch")
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    dq, dk, dv = (np.empty((B, N, H, D), np.float64) for _ in range(3))
    wt, wh, ww = window
    rc = _load().oracle_attend_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, D, T, Hg, Wg,
                                        wt, wh, ww, _BORDER[border], float(scale), _ptr(mask),
                                        _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attend_backward rejected its arguments (rc={rc})")
    return dq, dk, dv


def backward_dq_rows(q, k, v, dout, grid, window, scale, mask, rows, nthreads: int = 0,
                     border: str = "shift") -> np.ndarray:
    """dL/dQ of the listed rows: [len(rows), heads, D] float64."""
    q, k, v, dout = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, N, H, D = q.shape
    T, Hg, Wg = grid
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H, D), np.float64)
    wt, wh, ww = window
    rc = _load().oracle_attend_backward_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, D, T, Hg,
                                                Wg, wt, wh, ww, _BORDER[border], float(scale),
                                                _ptr(mask), _ptr(rows), rows.size, _ptr(out),
                                                int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attend_backward_dq_rows rejected its arguments (rc={rc})")
    return out


def backward_kv_rows(q, k, v, dout, grid, window, scale, mask, rows, heads=None, nthreads: int = 0,
                     border: str = "shift"):
    """dL/dK and dL/dV of the listed keys (rows = b*N + j, each once) for the
    listed heads (default: all): two float64 arrays [len(rows), len(heads), D]
    (oracle_attend_backward_kv_rows)."""
    q, k, v, dout = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    B, N, H, D = q.shape
    T, Hg, Wg = grid
    if T * Hg * Wg != N or any(x.shape != q.shape for x in (k, v, dout)):
        raise ValueError("shape mismatch")
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    hsel = np.ascontiguousarray(np.arange(H) if heads is None else heads, dtype=np.int32)
    dk = np.empty((rows.size, hsel.size, D), np.float64)
    dv = np.empty((rows.size, hsel.size, D), np.float64)
    wt, wh, ww = window
    rc = _load().oracle_attend_backward_kv_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, D, T, Hg, Wg,
                                                wt, wh, ww, _BORDER[border], float(scale), _ptr(mask),
                                                _ptr(rows), rows.size, _ptr(hsel), hsel.size, _ptr(dk), _ptr(dv),
                                                int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_attend_backward_kv_rows rejected its arguments (rc={rc})")
    return dk, dv
