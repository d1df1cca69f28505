"""Pins of the oracle's backward pass (dQ, dK, dV of heterogeneous attention).

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): the dense (Eq. 2) and local (Eq. 3) softmax attention
merged by Eq. 13, differentiated with the route held fixed.  The paper's
second training stage fine-tunes through this layer (§4, Training Setting).

Pins: central finite differences of the (separately pinned) oracle forward;
torch autograd in float64 through a brute-force masked softmax built from an
independent characterisation of each key set; sum identities that hold at
any size (sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per sample and head);
equal keys give dQ = 0.
"""
import itertools

import numpy as np
import pytest
import torch


def quantised(rng, shape, step=2.0 ** -6):
    """float32 values on a grid of `step`, so that x +- 2^-12 is exact."""
    return (np.round(rng.standard_normal(shape) / step) * step).astype(np.float32)


def allowed_matrix(grid, window, mask_row, border):
    """[N, N] key sets: all keys for dense rows; for local rows the window,
    described per axis by distance (cut) or as the nearest in-grid interval of
    length min(k, S) containing the position (shifted)."""
    T, H, W = grid
    N = T * H * W
    coords = np.array(list(itertools.product(range(T), range(H), range(W))))
    ext = np.array(grid)
    allowed = np.zeros((N, N), bool)
    for n in range(N):
        if mask_row[n] == 0:
            allowed[n] = True
            continue
        ok = np.ones(N, bool)
        for ax in range(3):
            S, k, p = ext[ax], window[ax], coords[n, ax]
            if border == "cut":
                ok &= np.abs(coords[:, ax] - p) <= (k - 1) // 2
            else:
                L = min(k, S)
                best = min((abs(s + (L - 1) / 2.0 - p), s) for s in range(S - L + 1) if s <= p < s + L)[1]
                ok &= (coords[:, ax] >= best) & (coords[:, ax] < best + L)
        allowed[n] = ok
    return allowed


def torch_grads(q, k, v, dout, grid, window, scale, mask, border):
    B, N, H, D = q.shape
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    outs = []
    for b in range(B):
        allowed = torch.from_numpy(allowed_matrix(grid, window, mask[b], border))
        for h in range(H):
            s = scale * tq[b, :, h, :] @ tk[b, :, h, :].T
            s = s.masked_fill(~allowed, float("-inf"))
            outs.append((torch.softmax(s, dim=1) @ tv[b, :, h, :], b, h))
    loss = sum((o * torch.from_numpy(dout[b, :, h, :].astype(np.float64))).sum() for o, b, h in outs)
    loss.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("border", ["shift", "cut"])
@pytest.mark.parametrize("grid,window", [((3, 4, 5), (3, 3, 3)), ((2, 5, 6), (1, 3, 5))])
def test_backward_matches_torch_autograd(oracle_mod, border, grid, window):
    rng = np.random.default_rng(sum(grid) + (border == "cut"))
    N = int(np.prod(grid))
    q, k, v, do = (rng.standard_normal((2, N, 2, 8)).astype(np.float32) for _ in range(4))
    mask = (rng.random((2, N)) < 0.7).astype(np.uint8)
    dq, dk, dv = oracle_mod.backward(q, k, v, do, grid, window, 0.4, mask, border=border)
    rq, rk, rv = torch_grads(q, k, v, do, grid, window, 0.4, mask, border)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("border", ["shift", "cut"])
def test_backward_matches_finite_differences(oracle_mod, border):
    """dL/dx for L = sum(dO * O) by central differences of the oracle forward."""
    grid, window, scale = (2, 3, 4), (1, 3, 3), 0.5
    rng = np.random.default_rng(11)
    N = 24
    q, k, v, do = (quantised(rng, (1, N, 2, 4)) for _ in range(4))
    mask = (rng.random((1, N)) < 0.6).astype(np.uint8)
    dq, dk, dv = oracle_mod.backward(q, k, v, do, grid, window, scale, mask, border=border)

    def loss(qq, kk, vv):
        o = oracle_mod.forward(qq, kk, vv, grid, window, scale, mask, border=border)
        return float((o * do.astype(np.float64)).sum())

    h = 2.0 ** -12
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in itertools.product(range(N), range(2), range(4)):
            if (idx[0] * 8 + idx[1] * 4 + idx[2]) % 5:
                continue  # a fifth of the elements, spread over tokens, heads and dims
            args = [q.copy(), k.copy(), v.copy()]
            args[which][(0,) + idx] += np.float32(h)
            up = loss(*args)
            args[which][(0,) + idx] -= np.float32(2 * h)
            down = loss(*args)
            fd = (up - down) / (2 * h)
            assert abs(fd - grad[(0,) + idx]) < 1e-6, (which, idx, fd, grad[(0,) + idx])


def test_backward_sum_identities_and_rows(oracle_mod):
    grid, window = (6, 10, 20), (3, 7, 7)
    N = 1200
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((2, N, 2, 32)).astype(np.float32) for _ in range(4))
    mask = (rng.random((2, N)) < 0.8).astype(np.uint8)
    dq, dk, dv = oracle_mod.backward(q, k, v, do, grid, window, 0.17, mask)
    # each row's dS sums to zero, so the key gradients of a (sample, head) do
    scale_k = np.abs(dk).sum(axis=1).max()
    assert np.abs(dk.sum(axis=1)).max() < 1e-12 * scale_k * N
    # each row's weights sum to one, so dV sums to dO
    np.testing.assert_allclose(dv.sum(axis=1), do.astype(np.float64).sum(axis=1), rtol=1e-11, atol=1e-10)
    rows = np.array([0, 17, 599, 1199, 1200, 2399], dtype=np.int64)
    got = oracle_mod.backward_dq_rows(q, k, v, do, grid, window, 0.17, mask, rows)
    np.testing.assert_array_equal(got, dq.reshape(2 * N, 2, 32)[rows])


def test_equal_keys_give_zero_dq(oracle_mod):
    grid, window = (2, 4, 4), (1, 3, 3)
    N = 32
    rng = np.random.default_rng(2)
    q, v, do = (rng.standard_normal((1, N, 1, 8)).astype(np.float32) for _ in range(3))
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, 8)).astype(np.float32), (1, N, 1, 8)).copy()
    mask = (rng.random((1, N)) < 0.5).astype(np.uint8)
    dq, _, _ = oracle_mod.backward(q, k, v, do, grid, window, 1.0, mask)
    assert np.abs(dq).max() < 1e-14


@pytest.mark.parametrize("border", ["shift", "cut"])
@pytest.mark.parametrize("grid,window", [((3, 4, 5), (3, 3, 3)), ((2, 5, 6), (1, 3, 5))])
def test_kv_rows_match_torch_autograd(oracle_mod, border, grid, window):
    """dK, dV of listed keys and heads against torch autograd through the
    brute-force masked softmax (every key of both samples, heads reordered)."""
    rng = np.random.default_rng(3 * sum(grid) + (border == "cut"))
    N = int(np.prod(grid))
    q, k, v, do = (rng.standard_normal((2, N, 3, 8)).astype(np.float32) for _ in range(4))
    mask = (rng.random((2, N)) < 0.7).astype(np.uint8)
    rows = rng.permutation(2 * N).astype(np.int64)
    heads = [2, 0]
    dk, dv = oracle_mod.backward_kv_rows(q, k, v, do, grid, window, 0.4, mask, rows, heads=heads, border=border)
    _, rk, rv = torch_grads(q, k, v, do, grid, window, 0.4, mask, border)
    rk = rk.reshape(2 * N, 3, 8)[rows][:, heads]
    rv = rv.reshape(2 * N, 3, 8)[rows][:, heads]
    np.testing.assert_allclose(dk, rk, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, rv, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("border", ["shift", "cut"])
def test_kv_rows_equal_full_backward(oracle_mod, border):
    """On a 1200-token grid with borders in every axis: the listed keys' rows
    of the full backward, whichever sample and head."""
    grid, window = (6, 10, 20), (3, 7, 9)
    N = 1200
    rng = np.random.default_rng(17 + (border == "cut"))
    q, k, v, do = (rng.standard_normal((2, N, 2, 16)).astype(np.float32) for _ in range(4))
    mask = (rng.random((2, N)) < 0.8).astype(np.uint8)
    _, fk, fv = oracle_mod.backward(q, k, v, do, grid, window, 0.21, mask, border=border)
    rows = np.array([0, 19, 180, 599, 1199, 1200, 1201, 1719, 2399, 1500], dtype=np.int64)
    dk, dv = oracle_mod.backward_kv_rows(q, k, v, do, grid, window, 0.21, mask, rows, heads=[1], border=border)
    np.testing.assert_allclose(dk[:, 0], fk.reshape(2 * N, 2, 16)[rows, 1], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dv[:, 0], fv.reshape(2 * N, 2, 16)[rows, 1], rtol=1e-10, atol=1e-13)


def test_kv_rows_closed_forms(oracle_mod):
    """All keys equal and all values equal: every weight is 1/|key set| and
    dP_j is the same for every key, so dS = 0, dK = 0 and dV_j = sum over the
    rows that see j of dO_n / |key set of n|."""
    grid, window = (2, 4, 4), (1, 3, 3)
    N = 32
    rng = np.random.default_rng(9)
    q, do = (rng.standard_normal((1, N, 1, 8)).astype(np.float32) for _ in range(2))
    k, v = (np.broadcast_to(rng.standard_normal((1, 1, 1, 8)).astype(np.float32), (1, N, 1, 8)).copy()
            for _ in range(2))
    mask = (rng.random((1, N)) < 0.5).astype(np.uint8)
    rows = np.arange(N, dtype=np.int64)
    dk, dv = oracle_mod.backward_kv_rows(q, k, v, do, grid, window, 1.0, mask, rows)
    assert np.abs(dk).max() < 1e-13
    allowed = allowed_matrix(grid, window, mask[0], "shift")
    expect = (allowed / allowed.sum(axis=1, keepdims=True)).T @ do[0, :, 0, :].astype(np.float64)
    np.testing.assert_allclose(dv[:, 0], expect, rtol=1e-12, atol=1e-14)


def test_kv_rows_rejects_bad_lists(oracle_mod):
    grid, window = (2, 3, 4), (1, 3, 3)
    q = np.zeros((1, 24, 2, 4), np.float32)
    mask = np.ones((1, 24), np.uint8)
    for rows, heads in (([3, 3], None), ([24], None), ([-1], None), ([1], [2]), ([1], [])):
        with pytest.raises(ValueError):
            oracle_mod.backward_kv_rows(q, q, q, q, grid, window, 1.0, mask, np.array(rows), heads=heads)
