"""The C ABI of include/hetattn.h: symbols, version, status strings and the
host-side argument checks.  Nothing here launches a kernel: every call below
is rejected on the host before any HIP call, so these run without a GPU."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import uncertainty_routed_heterogeneous_amd as het

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hetattn.h")
FAKE = 0x1000  # never dereferenced: each call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(het_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(het.LIB_PATH):
        import uncertainty_routed_heterogeneous_amd.build as b
        b.build()
    return het.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names == sorted(het.SIGNATURES), "binding and header disagree"
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.het_attn_abi_version() == het.ABI_VERSION == 5
    for st in range(5):
        assert het.status_string(st)
    assert het.status_string(99) == "unknown status"


def good_shape(**kw):
    d = dict(batch=1, heads=2, head_dim=64, grid=(4, 8, 8), window=(3, 3, 3), dtype=het.HET_F32)
    border = kw.pop("border", None)
    d.update(kw)
    s = het.make_shape(d["batch"], d["heads"], d["head_dim"], d["grid"], d["window"], d["dtype"])
    if border is not None:
        s.border = border
    return s


def fake_route():
    return het.RouteStruct(FAKE, FAKE, FAKE, FAKE, FAKE, -1)


def call_route(lib, shape, mode=het.HET_TOP_RHO, param=0.2, u=FAKE, route=None, ws=None, ws_bytes=0):
    r = route if route is not None else fake_route()
    return lib.het_attn_route(ctypes.byref(shape) if shape is not None else None, u, mode, param,
                              ctypes.byref(r), ws, ws_bytes, None)


def call_forward(lib, shape, route=None, q=FAKE, o=FAKE, ws=None, ws_bytes=0):
    r = route if route is not None else fake_route()
    return lib.het_attn_forward(ctypes.byref(shape) if shape is not None else None, q, FAKE, FAKE,
                                ctypes.byref(r), o, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,status", [
    (dict(batch=0), het.HET_ERR_INVALID_ARG),
    (dict(heads=-1), het.HET_ERR_INVALID_ARG),
    (dict(grid=(0, 8, 8)), het.HET_ERR_INVALID_ARG),
    (dict(window=(2, 3, 3)), het.HET_ERR_INVALID_ARG),
    (dict(window=(3, 3, 0)), het.HET_ERR_INVALID_ARG),
    (dict(dtype=7), het.HET_ERR_INVALID_ARG),
    (dict(border=2), het.HET_ERR_INVALID_ARG),
    (dict(border=-1), het.HET_ERR_INVALID_ARG),
    (dict(head_dim=96), het.HET_ERR_UNSUPPORTED),
    (dict(head_dim=256), het.HET_ERR_UNSUPPORTED),
    (dict(grid=(64, 64, 64), heads=64, head_dim=128, batch=8), het.HET_ERR_UNSUPPORTED),
    (dict(grid=(4, 8, 64), window=(3, 3, 27)), het.HET_ERR_UNSUPPORTED),
])
def test_shape_errors(lib, bad, status):
    s = good_shape(**bad)
    assert call_route(lib, s) == status
    assert call_forward(lib, s) == status
    assert lib.het_attn_workspace_bytes(ctypes.byref(s)) == 0
    assert lib.het_attn_route_workspace_bytes(ctypes.byref(s)) == 0


def test_null_and_bad_scale(lib):
    assert call_route(lib, None) == het.HET_ERR_INVALID_ARG
    assert call_forward(lib, None) == het.HET_ERR_INVALID_ARG
    s = good_shape()
    s.scale = float("nan")
    assert call_route(lib, s) == het.HET_ERR_INVALID_ARG
    s.scale = float("inf")
    assert call_forward(lib, s) == het.HET_ERR_INVALID_ARG


def test_route_argument_errors(lib):
    s = good_shape()
    assert call_route(lib, s, u=None) == het.HET_ERR_INVALID_ARG
    for field in ("mask", "dense_idx", "local_idx", "counts", "thresh"):
        r = fake_route()
        setattr(r, field, None)
        assert call_route(lib, s, route=r) == het.HET_ERR_INVALID_ARG, field
    for rho in (-0.01, 1.01, float("nan"), float("inf")):
        assert call_route(lib, s, het.HET_TOP_RHO, rho) == het.HET_ERR_INVALID_ARG
    for c in (float("nan"), float("inf"), float("-inf")):
        assert call_route(lib, s, het.HET_MEAN_STD, c) == het.HET_ERR_INVALID_ARG
    assert call_route(lib, s, mode=5) == het.HET_ERR_INVALID_ARG
    # u may be NULL only for the uniform lattice, which still checks rho
    for mode in (het.HET_TOP_RHO, het.HET_MEAN_STD):
        assert call_route(lib, s, mode, 0.2, u=None) == het.HET_ERR_INVALID_ARG
    for rho in (-0.5, 1.5, float("nan")):
        assert call_route(lib, s, het.HET_UNIFORM, rho, u=None) == het.HET_ERR_INVALID_ARG
    r = fake_route()
    r.local_idx = None
    assert call_route(lib, s, het.HET_UNIFORM, 0.2, u=None, route=r) == het.HET_ERR_INVALID_ARG


def test_forward_argument_errors(lib):
    s = good_shape()
    assert call_forward(lib, s, q=None) == het.HET_ERR_INVALID_ARG
    assert call_forward(lib, s, o=None) == het.HET_ERR_INVALID_ARG
    r = fake_route()
    r.dense_count_host = 257  # N = 256
    assert call_forward(lib, s, route=r) == het.HET_ERR_INVALID_ARG
    r.dense_count_host = -2
    assert call_forward(lib, s, route=r) == het.HET_ERR_INVALID_ARG
    r = fake_route()
    r.counts = None
    assert call_forward(lib, s, route=r) == het.HET_ERR_INVALID_ARG


def test_workspace_size(lib):
    assert lib.het_attn_workspace_bytes(None) == 0
    assert lib.het_attn_workspace_bytes(ctypes.byref(good_shape())) >= 0


def route_ws_expected(batch: int, n: int) -> int:
    """The top-rho route's workspace as documented: per sample, two
    [G][1024] arrays, [G] counts and [G][2056] candidate lists of 64-bit
    tagged words (G = ceil(N / 2048) workgroups), rounded up to 256 bytes;
    none below 8192 tokens, above 128 workgroups per sample or 1024 per
    launch."""
    g = -(-n // 2048)
    if n < 8192 or g > 128 or batch * g > 1024:
        return 0
    per = (2 * g * 1024 + g + g * 2056) * 8
    return batch * (-(-per // 256) * 256)


@pytest.mark.parametrize("batch,grid", [(1, (4, 8, 8)), (1, (4, 32, 63)), (1, (4, 32, 64)),
                                        (1, (21, 30, 52)), (2, (31, 22, 40)), (1, (39, 40, 41)),
                                        (1, (64, 64, 64)), (1, (64, 64, 65)), (8, (64, 64, 64)),
                                        (64, (21, 30, 52)), (65, (21, 30, 52))])
def test_route_workspace_size(lib, batch, grid):
    s = good_shape(batch=batch, grid=grid, head_dim=128, heads=1)
    got = lib.het_attn_route_workspace_bytes(ctypes.byref(s))
    assert got == route_ws_expected(batch, math.prod(grid))
    assert lib.het_attn_route_workspace_bytes(None) == 0


def test_route_workspace_errors(lib):
    # 21x30x52 tokens: the top-rho route runs over 16 workgroups per sample.
    s = good_shape(grid=(21, 30, 52), head_dim=128, heads=1)
    need = lib.het_attn_route_workspace_bytes(ctypes.byref(s))
    assert need > 0
    assert call_route(lib, s) == het.HET_ERR_WORKSPACE
    assert call_route(lib, s, ws=FAKE, ws_bytes=need - 1) == het.HET_ERR_WORKSPACE
    assert call_route(lib, s, ws=None, ws_bytes=need) == het.HET_ERR_WORKSPACE
    # argument errors still come first
    assert call_route(lib, s, param=1.5) == het.HET_ERR_INVALID_ARG


def test_binding_rejects_bad_tensors():
    import torch
    u = torch.zeros(1, 256)
    with pytest.raises(ValueError):
        het.route(u, (4, 8, 8), (3, 3, 3), 2, 64, torch.float32, rho=0.2)  # not on a GPU
    with pytest.raises(ValueError):
        het.route(u, (4, 8, 8), (3, 3, 3), 2, 64, torch.float32)  # neither rho nor c


def cpu_route(B, grid, window=(3, 3, 3)):
    """A Route of CPU tensors: the binding's shape checks run before any
    device check, so each mismatch below is rejected without a GPU."""
    import torch
    N = int(np.prod(grid))
    return het.Route(torch.zeros((B, N), dtype=torch.uint8), torch.zeros((B, N), dtype=torch.int32),
                     torch.zeros((B, N), dtype=torch.int32), torch.zeros((B, 2), dtype=torch.int32),
                     torch.zeros(B, dtype=torch.float64), -1, tuple(grid), tuple(window))


@pytest.mark.parametrize("case", ["grid_vs_N", "batch_vs_route", "kv_shape", "kv_dtype", "not_4d",
                                  "not_contiguous", "o_shape", "dout_dtype", "counts_shape", "cpu_tensors"])
def test_binding_rejects_mismatched_shapes(case):
    """A route made for another layer shape would send the kernels outside
    the tensors (they size every index from the grid and the route's
    buffers), so the binding refuses it before any launch."""
    import torch
    B, grid, H, D = 2, (2, 3, 4), 2, 64
    N = 24
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16)
    k, v, o, do = (torch.zeros_like(q) for _ in range(4))
    r = cpu_route(B, grid)
    if case == "grid_vs_N":
        r = cpu_route(B, (2, 3, 5))
    elif case == "batch_vs_route":
        r = cpu_route(1, grid)
    elif case == "kv_shape":
        k = torch.zeros((B, N, H + 1, D), dtype=torch.bfloat16)
    elif case == "kv_dtype":
        v = torch.zeros_like(q, dtype=torch.float32)
    elif case == "not_4d":
        q, k, v = (x.reshape(B, N, H * D) for x in (q, k, v))
    elif case == "not_contiguous":
        q = torch.zeros((B, N, D, H), dtype=torch.bfloat16).transpose(2, 3)
    elif case == "o_shape":
        o = torch.zeros((B, N - 1, H, D), dtype=torch.bfloat16)
    elif case == "dout_dtype":
        do = torch.zeros_like(q, dtype=torch.float32)
    elif case == "counts_shape":
        r.counts = torch.zeros((B, 3), dtype=torch.int32)
    with pytest.raises(ValueError):
        het.backward(q, k, v, r, o, do)
    if case not in ("o_shape", "dout_dtype"):
        with pytest.raises(ValueError):
            het.forward(q, k, v, r)


def test_binding_rejects_bad_outputs():
    import torch
    B, grid, H, D = 1, (2, 3, 4), 2, 64
    q = torch.zeros((B, 24, H, D), dtype=torch.bfloat16)
    r = cpu_route(B, grid)
    for out in (torch.zeros((B, 24, H, D), dtype=torch.float32), torch.zeros((B, 24, H, 2 * D))[..., ::2],
                torch.zeros((B, 23, H, D), dtype=torch.bfloat16)):
        with pytest.raises(ValueError):
            het.forward(q, q, q, r, out=out)
        with pytest.raises(ValueError):
            het.backward(q, q, q, r, q, q, out=(out, torch.zeros_like(q), torch.zeros_like(q)))
    with pytest.raises(ValueError):
        het.backward(q, q, q, r, q, q, out=(torch.zeros_like(q), torch.zeros_like(q)))


def call_swap(lib, shape, src=None, dst=None, r=0.07, n_blocks=1):
    s_in = src if src is not None else fake_route()
    s_out = dst if dst is not None else het.RouteStruct(0x100000, 0x200000, 0x300000, 0x400000,
                                                         0x500000, -1)
    return lib.het_attn_swap(ctypes.byref(shape) if shape is not None else None,
                             ctypes.byref(s_in) if s_in is not False else None, r, 7, 0, 0,
                             n_blocks, ctypes.byref(s_out) if s_out is not False else None, None)


def test_swap_argument_errors(lib):
    s = good_shape()  # N = 256
    assert call_swap(lib, None) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, src=False) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, dst=False) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, good_shape(head_dim=96)) == het.HET_ERR_UNSUPPORTED
    r = fake_route()
    r.mask = None
    assert call_swap(lib, s, src=r) == het.HET_ERR_INVALID_ARG
    for field in ("mask", "dense_idx", "local_idx", "counts"):
        d = het.RouteStruct(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, -1)
        setattr(d, field, None)
        assert call_swap(lib, s, dst=d) == het.HET_ERR_INVALID_ARG, field
    for ratio in (-0.01, 1.01, float("nan"), float("inf")):
        assert call_swap(lib, s, r=ratio) == het.HET_ERR_INVALID_ARG
    for nb in (0, -1, 65536):
        assert call_swap(lib, s, n_blocks=nb) == het.HET_ERR_INVALID_ARG
    r = fake_route()
    r.dense_count_host = 257
    assert call_swap(lib, s, src=r) == het.HET_ERR_INVALID_ARG


def test_swap_overlap_errors(lib):
    """Outputs may not overlap the input mask or thresholds, except for the
    in-place form (one route, the very same buffers)."""
    s = good_shape()  # B = 1, N = 256
    src = het.RouteStruct(0x10000, 0x20000, 0x30000, 0x40000, 0x50000, -1)

    def dst(**kw):
        d = het.RouteStruct(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, -1)
        for k, v in kw.items():
            setattr(d, k, v)
        return d

    # The same mask with two routes: route 1 would overwrite what route 0 reads.
    assert call_swap(lib, s, src, dst(mask=0x10000), n_blocks=2) == het.HET_ERR_INVALID_ARG
    # Index lists, counts or thresholds on top of the input mask.
    assert call_swap(lib, s, src, dst(dense_idx=0x10000 - 512)) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, src, dst(local_idx=0x10000 + 255)) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, src, dst(counts=0x10000 + 100)) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, src, dst(thresh=0x10000 + 8)) == het.HET_ERR_INVALID_ARG
    # A mask shifted into the input mask, and thresholds shared by two routes.
    assert call_swap(lib, s, src, dst(mask=0x10000 + 1)) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, src, dst(thresh=0x50000), n_blocks=2) == het.HET_ERR_INVALID_ARG
    assert call_swap(lib, s, src, dst(mask=0x50000 + 4)) == het.HET_ERR_INVALID_ARG


def test_route_random_argument_errors(lib):
    s = good_shape()

    def call(shape=s, rho=0.2, n_blocks=1, out=None):
        o = out if out is not None else het.RouteStruct(0x100000, 0x200000, 0x300000, 0x400000, 0, -1)
        return lib.het_attn_route_random(ctypes.byref(shape) if shape is not None else None, rho, 1, 0, 0,
                                         n_blocks, ctypes.byref(o) if o is not False else None, None)

    assert call(shape=None) == het.HET_ERR_INVALID_ARG
    assert call(shape=good_shape(window=(4, 3, 3))) == het.HET_ERR_INVALID_ARG
    assert call(out=False) == het.HET_ERR_INVALID_ARG
    for rho in (-0.01, 1.01, float("nan")):
        assert call(rho=rho) == het.HET_ERR_INVALID_ARG
    for nb in (0, -3, 65536):
        assert call(n_blocks=nb) == het.HET_ERR_INVALID_ARG
    for field in ("mask", "dense_idx", "local_idx", "counts"):
        o = het.RouteStruct(0x100000, 0x200000, 0x300000, 0x400000, 0, -1)
        setattr(o, field, None)
        assert call(out=o) == het.HET_ERR_INVALID_ARG, field


def test_backward_argument_errors(lib):
    s = good_shape()  # B=1, N=256, heads=2, D=64, f32: 128 KiB per tensor
    ws_n = lib.het_attn_backward_workspace_bytes(ctypes.byref(s))
    assert ws_n == 2 * 1 * 2 * 256 * 4 + 4 * 1024 * 256 * 4
    assert lib.het_attn_backward_workspace_bytes(ctypes.byref(good_shape(head_dim=96))) == 0
    span = 1 << 20
    base = {n: (i + 1) * span for i, n in enumerate(("q", "k", "v", "o", "dout", "dq", "dk", "dv", "ws"))}

    def call(shape=s, route=None, ws_bytes=ws_n, **kw):
        p = dict(base, **kw)
        r = route if route is not None else fake_route()
        return lib.het_attn_backward(ctypes.byref(shape) if shape is not None else None, p["q"], p["k"],
                                     p["v"], ctypes.byref(r), p["o"], p["dout"], p["dq"], p["dk"], p["dv"],
                                     p["ws"], ws_bytes, None)

    assert call(shape=None) == het.HET_ERR_INVALID_ARG
    assert call(shape=good_shape(head_dim=96)) == het.HET_ERR_UNSUPPORTED
    assert call(shape=good_shape(grid=(1, 1, 40000), window=(1, 1, 1))) == het.HET_ERR_UNSUPPORTED
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        assert call(**{name: None}) == het.HET_ERR_INVALID_ARG, name
    r = fake_route()
    r.counts = None
    assert call(route=r) == het.HET_ERR_INVALID_ARG
    r = fake_route()
    r.dense_count_host = 300
    assert call(route=r) == het.HET_ERR_INVALID_ARG
    # outputs overlapping an input or each other
    assert call(dq=base["v"] + 64) == het.HET_ERR_INVALID_ARG
    assert call(dk=base["dq"] + 4096) == het.HET_ERR_INVALID_ARG
    assert call(dv=base["dout"]) == het.HET_ERR_INVALID_ARG
    # workspace
    assert call(ws_bytes=ws_n - 1) == het.HET_ERR_WORKSPACE
    assert call(ws=None) == het.HET_ERR_WORKSPACE


def test_lse_entry_points_argument_errors(lib):
    """The forms that hand the rows' LSE from the forward to the backward: a
    NULL LSE is an argument error, and fp32 inputs are not supported (both
    found before any device call)."""
    s = good_shape()
    r = fake_route()
    args = (ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(r), FAKE)
    assert lib.het_attn_forward_lse(*args, None, None, 0, None) == het.HET_ERR_INVALID_ARG
    assert lib.het_attn_backward_lse(*args, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == het.HET_ERR_INVALID_ARG
    s32 = good_shape()
    s32.dtype = het.HET_F32
    args32 = (ctypes.byref(s32), FAKE, FAKE, FAKE, ctypes.byref(r), FAKE)
    assert lib.het_attn_forward_lse(*args32, FAKE + 4096, None, 0, None) == het.HET_ERR_UNSUPPORTED
