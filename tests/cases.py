"""Destination patterns shared by the GPU parity tests (input generation only)."""
import numpy as np


def heavy_destinations(E, N, seed):
    """About 40 % of the edges on 1 % of the nodes (at least 3, always including
    nodes 0 and N - 1), spread over the whole id range, the rest uniform; edge
    order random.  The heavy nodes then have far more than 1.5x the mean
    degree."""
    rng = np.random.default_rng(seed)
    n_heavy = max(3, N // 100)
    heavy = np.unique(np.concatenate([rng.choice(N, n_heavy, replace=False), [0, N - 1]]))
    dst = rng.integers(0, N, E)
    pick = rng.random(E) < 0.4
    dst[pick] = heavy[rng.integers(0, len(heavy), int(pick.sum()))]
    return dst.astype(np.int64)
