"""Pins of the oracle's per-block random swap and of its generator.

[HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient Video
Diffusion" (HetA-DiT): the swap of uncertain and certain tokens at each block
(§3.2.2, after Eq. 12) and its ratio r (App. B, Random Token Percentage,
Table 8).  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11.
"""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def test_philox_known_answers(oracle_mod):
    # Known-answer vectors published with the Philox authors' reference
    # library (Random123), for philox4x32 with 10 rounds.
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in cases:
        assert oracle_mod.philox4x32_10(ctr, key) == want


def keys_of(oracle_mod, B, N, seed, step, block):
    key = (seed & 0xFFFFFFFF, seed >> 32)
    return np.array([[oracle_mod.philox4x32_10((i, b, block, step), key)[0] for i in range(N)]
                     for b in range(B)], dtype=np.uint64)


def base_route(oracle_mod, B=2, N=300, rho=0.2, seed=3):
    u = np.random.default_rng(seed).random((B, N)).astype(np.float32)
    return oracle_mod.route_top_rho(u, rho)


def check_route_consistent(r):
    B, N = r.mask.shape
    for b in range(B):
        nd, nl = r.counts[b]
        assert nd + nl == N
        d = r.dense_idx[b, :nd]
        l = r.local_idx[b, :nl]
        assert np.all(np.diff(d) > 0) and np.all(np.diff(l) > 0)
        assert np.all(r.dense_idx[b, nd:] == -1) and np.all(r.local_idx[b, nl:] == -1)
        assert np.all(r.mask[b, d] == 0) and np.all(r.mask[b, l] == 1)


def test_zero_ratio_is_identity(oracle_mod):
    r0 = base_route(oracle_mod)
    s = oracle_mod.route_swap(r0.mask, 0.0, 123, 4, 5)
    np.testing.assert_array_equal(s.mask, r0.mask)
    np.testing.assert_array_equal(s.dense_idx, r0.dense_idx)
    np.testing.assert_array_equal(s.counts, r0.counts)


@pytest.mark.parametrize("r", [0.01, 0.07, 0.15])
def test_counts_kept_and_exactly_s_each_way(oracle_mod, r):
    r0 = base_route(oracle_mod)
    s = oracle_mod.route_swap(r0.mask, r, 99, 1, 2)
    check_route_consistent(s)
    np.testing.assert_array_equal(s.counts, r0.counts)
    N = r0.mask.shape[1]
    S = int(np.floor(r * N + 0.5))
    for b in range(r0.mask.shape[0]):
        out = np.sum((r0.mask[b] == 0) & (s.mask[b] == 1))
        inn = np.sum((r0.mask[b] == 1) & (s.mask[b] == 0))
        assert out == inn == min(S, r0.counts[b, 0], r0.counts[b, 1])


def test_swap_count_rounds_half_up(oracle_mod):
    """S = floor(r*N + 1/2): r*N = 21.7 at N = 310 gives 22, and 2.5 at N = 50
    (r = 0.05) gives 3."""
    for N, r, S in [(310, 0.07, 22), (50, 0.05, 3), (300, 0.07, 21)]:
        r0 = base_route(oracle_mod, B=1, N=N, rho=0.3)
        s = oracle_mod.route_swap(r0.mask, r, 8, 0, 0)
        assert np.sum((r0.mask[0] == 0) & (s.mask[0] == 1)) == S


def test_swapped_tokens_have_the_smallest_keys(oracle_mod):
    """In each set the swapped tokens are the S with the smallest Philox key
    (ties by index): every swapped key is below every kept key of its set."""
    B, N, seed, step, block = 2, 300, 0x1234_5678_9ABC, 7, 11
    r0 = base_route(oracle_mod, B, N)
    s = oracle_mod.route_swap(r0.mask, 0.07, seed, step, block)
    keys = keys_of(oracle_mod, B, N, seed, step, block)
    idx = np.arange(N, dtype=np.uint64)
    rank = keys * np.uint64(1 << 20) + idx  # (key, index) order as one integer
    for b in range(B):
        for was_dense in (True, False):
            members = (r0.mask[b] == 0) if was_dense else (r0.mask[b] == 1)
            moved = members & (s.mask[b] != r0.mask[b])
            kept = members & ~moved
            assert moved.sum() == 21
            assert rank[b][moved].max() < rank[b][kept].min()


def test_ratio_at_rho_swaps_the_whole_dense_set(oracle_mod):
    """'20% (all)' of Table 8 at rho = 0.2: S = K, so no originally dense token
    stays dense and the new dense set is K random former local tokens."""
    r0 = base_route(oracle_mod, B=1, N=500, rho=0.2)
    s = oracle_mod.route_swap(r0.mask, 0.2, 5, 0, 0)
    assert np.all(s.mask[0][r0.mask[0] == 0] == 1)
    assert s.counts[0, 0] == r0.counts[0, 0] == 100


def test_swap_capped_by_the_smaller_set(oracle_mod):
    r0 = base_route(oracle_mod, B=1, N=400, rho=0.9)  # 360 dense, 40 local
    s = oracle_mod.route_swap(r0.mask, 0.5, 5, 0, 0)
    assert np.all(s.mask[0][r0.mask[0] == 1] == 0)  # all 40 local tokens became dense
    np.testing.assert_array_equal(s.counts, r0.counts)
    # and every sample edge: all dense / all local leave nothing to swap
    for rho in (0.0, 1.0):
        ra = base_route(oracle_mod, B=1, N=50, rho=rho)
        np.testing.assert_array_equal(oracle_mod.route_swap(ra.mask, 0.3, 1, 0, 0).mask, ra.mask)


def test_deterministic_and_keyed_by_block(oracle_mod):
    r0 = base_route(oracle_mod)
    a = oracle_mod.route_swap(r0.mask, 0.07, 42, 3, 8)
    b = oracle_mod.route_swap(r0.mask, 0.07, 42, 3, 8)
    np.testing.assert_array_equal(a.mask, b.mask)
    for other in [(42, 3, 9), (42, 4, 8), (43, 3, 8)]:
        assert not np.array_equal(oracle_mod.route_swap(r0.mask, 0.07, *other).mask, a.mask)


def test_uniform_coverage_over_blocks(oracle_mod):
    """Each certain token is drawn with probability p = S/(N-K) per block, so
    over B blocks it reaches dense attention at least once with probability
    1-(1-p)^B (App. B's coverage argument with the per-set fraction; with
    r = 0.07 and B = 30 the pages quote ~0.89 for p = r)."""
    w = W.WORKLOADS["wan13b"]
    u = W.make_u(w)
    r0 = oracle_mod.route_top_rho(u, 0.2)
    N = w.n_tokens
    K = int(r0.counts[0, 0])
    S = int(np.floor(0.07 * N + 0.5))
    p = S / (N - K)
    local0 = r0.mask[0] == 1
    hits = np.zeros(N, np.int64)
    blocks = 30
    for blk in range(blocks):
        s = oracle_mod.route_swap(r0.mask, 0.07, 2024, 17, blk)
        hits += (s.mask[0] == 0) & local0
    cover = np.mean(hits[local0] > 0)
    want = 1 - (1 - p) ** blocks
    assert abs(cover - want) < 0.01, (cover, want)
    # draws per token ~ Binomial(30, p): mean and variance
    mean = hits[local0].mean()
    assert abs(mean - blocks * p) < 0.02
    assert abs(hits[local0].var() - blocks * p * (1 - p)) < 0.1


def test_page_coverage_figure_and_this_reading():
    """App. B quotes a coverage of about 0.89 for r = 0.07 over B = 30 blocks,
    i.e. 1-(1-r)^B with a certain token drawn with probability r per block.
    Under this build's reading (S = round(rN) of the N - K certain tokens move
    per block) a certain token is drawn with p = r/(1-rho), so its coverage is
    higher: 0.936 at rho = 0.2 (test_uniform_coverage_over_blocks measures it
    on the oracle's swaps)."""
    with open(GOLDEN) as f:
        g = json.load(f)["random_swap_coverage"]
    r, blocks = g["r"], g["blocks"]
    assert abs(1 - (1 - r) ** blocks - g["coverage_approx"]) < 0.005
    p = r / (1 - 0.2)
    assert abs(1 - (1 - p) ** blocks - 0.936) < 0.001


def test_equal_draws_split_by_index(oracle_mod):
    """Two tokens with the same draw at the selection boundary: only the one
    with the lower index moves; one more swap slot moves both."""
    from swap_cases import tie_cases, tie_mask
    for case in tie_cases():
        m = tie_mask(oracle_mod, case)
        x = oracle_mod.swap_draws(case["N"], case["b"], case["seed"], case["step"], case["block"])
        i, j = case["i"], case["j"]
        assert i < j and x[i] == x[j] == case["draw"]
        assert int(np.count_nonzero(x < x[i])) == case["c"]
        side_before = m[0, i]
        r = oracle_mod.route_swap(m, case["r"], case["seed"], case["step"], case["block"])
        assert r.mask[0, i] != side_before and r.mask[0, j] == side_before
        assert r.counts[0, 0] == int(np.count_nonzero(m == 0))
        r2 = oracle_mod.route_swap(m, (case["c"] + 2) / case["N"], case["seed"], case["step"],
                                   case["block"])
        assert r2.mask[0, i] != side_before and r2.mask[0, j] != side_before
