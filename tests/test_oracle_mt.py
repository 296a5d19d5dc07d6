"""The oracle's K-thread variant (oracle/zs_oracle_mt.c, the all-cores CPU
baseline) is bitwise equal to the sequential oracle (CPU only)."""
import numpy as np
import pytest

import oracle
import synthetic
from cases import heavy_destinations


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


FRAMES = [
    # (name, N, E, C, destinations)
    ("uniform", 64, 2000, 32, "uniform"),
    ("heavy", 300, 20000, 24, "heavy"),
    ("empty_nodes", 500, 900, 8, "uniform"),     # most nodes have no edge
    ("c5", 40, 1500, 5, "uniform"),
]


@pytest.mark.parametrize("name,N,E,C,kind", FRAMES, ids=[f[0] for f in FRAMES])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_mt_matches_oracle(name, N, E, C, kind, threads):
    w = synthetic.custom(name, N, E, C, seed=3300 + E + C, envelope=True)
    x = synthetic.make_inputs(w)
    if kind == "heavy":
        x["dst"] = heavy_destinations(E, N, seed=E)
    mt = oracle.get_mt()
    ref = oracle.forward(x["coupling"], x["radial"], x["dst"], N)
    got = mt.forward(x["coupling"], x["radial"], x["dst"], N, threads)
    assert np.array_equal(_bits(got), _bits(ref))
    gc, gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    mgc, mgr = mt.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"], threads)
    assert np.array_equal(_bits(mgc), _bits(gc))
    assert np.array_equal(_bits(mgr), _bits(gr))


def test_mt_no_edges_and_bad_index():
    mt = oracle.get_mt()
    N, C = 7, 8
    empty = np.zeros(0, np.int64)
    out = mt.forward(np.zeros((0, 15), np.float32), np.zeros((0, 3, C), np.float32), empty, N, 4)
    assert np.all(_bits(out) == 0)
    with pytest.raises(oracle.OracleIndexError):
        mt.backward(np.zeros((N, 16, C), np.float32), np.zeros((2, 15), np.float32),
                    np.zeros((2, 3, C), np.float32), np.array([0, N], np.int64), 2)
