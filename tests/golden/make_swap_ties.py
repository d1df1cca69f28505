"""Writes swap_ties.json: cases where two tokens of one sample draw the same
32-bit value and the per-block swap has to split them, taking the lower token
index first (the tie rule of the swap; Philox4x32-10 draws as in the oracle).

For each (N, side) the script searches seeds 1, 2, ... for a pair i < j with
equal draws x, such that the set holding i and j can be made of i, j and every
token whose draw is below x (c tokens), with S = c + 1 <= N - (c + 2) so that
the other set does not cap S.  The stored ratio r = (c + 1) / N gives
floor(r*N + 1/2) = c + 1.  The mask is rebuilt from the draws by the tests.

Run from the repository root: python tests/golden/make_swap_ties.py
Calls only the oracle."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def find_case(N, side, step=0, block=0, b=0):
    for seed in range(1, 1000):
        x = oracle.swap_draws(N, b, seed, step, block)
        vals, counts = np.unique(x, return_counts=True)
        for v in vals[counts == 2]:
            c = int(np.count_nonzero(x < v))
            if c + 1 <= N - (c + 2):
                i, j = (int(t) for t in np.flatnonzero(x == v))
                return dict(N=N, side=side, seed=seed, step=step, block=block, b=b, i=i, j=j,
                            draw=int(v), c=c, r=(c + 1) / N)
    raise RuntimeError(f"no tie found for N={N}")


def main():
    oracle.build()
    cases = [find_case(65536, "dense"), find_case(65536, "local"), find_case(131072, "dense"),
             find_case(131072, "local", step=5, block=17)]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "swap_ties.json")
    with open(path, "w") as f:
        json.dump(cases, f, indent=1)
        f.write("\n")
    print(path, cases)


if __name__ == "__main__":
    main()
