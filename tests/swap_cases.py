"""Inputs for the per-block swap tests: the tie cases of
golden/swap_ties.json (written by golden/make_swap_ties.py from the oracle's
draws) and seeded random masks."""
from __future__ import annotations

import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def tie_cases() -> list[dict]:
    with open(os.path.join(HERE, "golden", "swap_ties.json")) as f:
        return json.load(f)


def tie_mask(oracle_mod, case: dict) -> np.ndarray:
    """[1, N] mask whose `side` set is i, j and every token drawing below x."""
    x = oracle_mod.swap_draws(case["N"], case["b"], case["seed"], case["step"], case["block"])
    members = x < np.uint32(case["draw"])
    members[[case["i"], case["j"]]] = True
    dense = members if case["side"] == "dense" else ~members
    return np.where(dense, 0, 1).astype(np.uint8)[None, :]


def random_mask(B: int, N: int, p_dense: float, seed: int, local_value: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    dense = rng.random((B, N)) < p_dense
    return np.where(dense, 0, local_value).astype(np.uint8)
