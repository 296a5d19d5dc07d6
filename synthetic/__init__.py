"""Seeded synthetic workloads for the GIE zonal scatter.

This module only draws random numbers and arranges them into the operator's
input layouts; it contains none of the operator's arithmetic. Both the CPU
oracle (under ``oracle/``) and the HIP path read their inputs from here, so
the two sides always see identical bytes.

Shapes and statistics follow deepmd-kit PR #6072 ("fused Triton zonal scatter
for the GIE head"), sections "What" and "Boundary and layout contract":
lmax = 3, so the padded node layout has 16 rows, the zonal coupling has 15
columns (rows 1..15) and the radial features have 3 degree slots of C
channels.  The edge counts 158002 / 647170 for the 1000 / 4096-atom frames
come from deepmd-kit PR #6106 (SO(2) edge-cohort backward), table of observed
runtime cohorts.  The real frames are perturbed diamond crystals with about
158 neighbours per atom; the recipes below stand in for them.

Every tensor is drawn from its own PCG64 stream, keyed by (seed, tag), so
changing one tensor's recipe never shifts another's values.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

ROWS = 16      # (lmax + 1)^2 padded rows per node, lmax = 3
ZONAL = 15     # rows 1..15 carry a zonal coupling column each
SLOTS = 3      # one radial slot per degree l = 1, 2, 3

_TAG_DST, _TAG_COUPLING, _TAG_ENV, _TAG_RADIAL, _TAG_GRAD, _TAG_SHUFFLE = range(6)


@dataclass(frozen=True)
class Workload:
    name: str
    n_nodes: int
    n_edges: int
    channels: int
    dst_kind: str          # "uniform" | "near_constant" | "skewed"
    envelope: bool         # coupling scaled by a per-edge cutoff-envelope factor U(0,1)
    seed: int
    grouped: bool = False  # edges ordered by destination (as a centre-major neighbour list
                           # gives them) instead of shuffled


# The five workloads.  "headline" is the 4096-atom frame the pages time.
WORKLOADS = {
    "tiny": Workload("tiny", 64, 2000, 32, "uniform", False, 20261202),
    "n1000": Workload("n1000", 1000, 158002, 32, "uniform", True, 20261203),
    "headline": Workload("headline", 4096, 647170, 32, "near_constant", True, 20261204),
    "skewed": Workload("skewed", 4096, 647170, 32, "skewed", True, 20261205),
    "large": Workload("large", 16384, 2600000, 64, "uniform", False, 20261206),
    # the headline shape with i.i.d. uniform destinations (Poisson degrees) instead
    # of near-constant ones
    "headline_uniform": Workload("headline_uniform", 4096, 647170, 32, "uniform", True, 20261207),
    # the headline frame (same seed, degrees and values) with its edges grouped by
    # destination: the CSR order is then the edge order
    "headline_grouped": Workload("headline_grouped", 4096, 647170, 32, "near_constant", True,
                                 20261204, grouped=True),
}


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag])))


def _near_constant_degrees(n_nodes: int, n_edges: int, seed: int) -> np.ndarray:
    """Every node gets floor(E/N) edges; E mod N seeded nodes get one more."""
    base, extra = divmod(n_edges, n_nodes)
    deg = np.full(n_nodes, base, dtype=np.int64)
    if extra:
        deg[_rng(seed, _TAG_DST).choice(n_nodes, extra, replace=False)] += 1
    return deg


def _skewed_degrees(n_nodes: int, n_edges: int, seed: int,
                    n_vacuum: int = 64, lam_lo: float = 40.0,
                    lam_hi: float = 275.0) -> np.ndarray:
    """Slab with vacuum: n_vacuum nodes of degree 0, the rest split evenly into
    Poisson(lam_lo) and Poisson(lam_hi) halves, then corrected one edge at a
    time (nodes drawn proportionally to their half's rate) to total exactly E."""
    rng = _rng(seed, _TAG_DST)
    order = rng.permutation(n_nodes)
    vacuum = order[:n_vacuum]
    rest = order[n_vacuum:]
    half = len(rest) // 2
    lo, hi = rest[:half], rest[half:]
    deg = np.zeros(n_nodes, dtype=np.int64)
    rate = np.zeros(n_nodes, dtype=np.float64)
    deg[lo] = rng.poisson(lam_lo, size=len(lo))
    deg[hi] = rng.poisson(lam_hi, size=len(hi))
    rate[lo], rate[hi] = lam_lo, lam_hi
    rate[vacuum] = 0.0
    p = rate / rate.sum()
    diff = n_edges - int(deg.sum())
    while diff != 0:
        picks = rng.choice(n_nodes, abs(diff), replace=True, p=p)
        if diff > 0:
            np.add.at(deg, picks, 1)
        else:
            for n in picks:
                if deg[n] > 0:
                    deg[n] -= 1
        diff = n_edges - int(deg.sum())
    assert deg[vacuum].sum() == 0
    return deg


def make_dst(w: Workload) -> np.ndarray:
    """Destination node per edge, int64, in random edge order (grouped by
    destination, in increasing node id, when ``w.grouped``)."""
    if w.n_edges == 0:
        return np.zeros(0, dtype=np.int64)
    if w.dst_kind == "uniform":
        dst = _rng(w.seed, _TAG_DST).integers(0, w.n_nodes, size=w.n_edges, dtype=np.int64)
        return np.sort(dst, kind="stable") if w.grouped else dst
    if w.dst_kind == "near_constant":
        deg = _near_constant_degrees(w.n_nodes, w.n_edges, w.seed)
    elif w.dst_kind == "skewed":
        deg = _skewed_degrees(w.n_nodes, w.n_edges, w.seed)
    else:
        raise ValueError(f"unknown dst_kind {w.dst_kind!r}")
    dst = np.repeat(np.arange(w.n_nodes, dtype=np.int64), deg)
    return dst if w.grouped else dst[_rng(w.seed, _TAG_SHUFFLE).permutation(w.n_edges)]


def make_inputs(w: Workload | str, with_grad: bool = True, tiled_radial: bool = False) -> dict:
    """All operator inputs for workload ``w`` as contiguous numpy arrays.

    dst      (E,)          int64
    env      (E,)          float32, U(0,1) per-edge cutoff envelope factor
    coupling (E, 15)       float32, U(-1,1) (times env when the workload has one)
    radial   (E, 3, C)     float32, N(0,1)
    grad_out (N, 16, C)    float32, N(0,1)   (upstream gradient of the output)

    With ``tiled_radial`` the radial tensor is not materialised: ``radial_pool``
    holds the pool it tiles (see ``radial_pool``) instead.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    E, N, C = w.n_edges, w.n_nodes, w.channels
    out = {"workload": w, "dst": make_dst(w)}
    env = _rng(w.seed, _TAG_ENV).uniform(0.0, 1.0, size=E)
    cpl = _rng(w.seed, _TAG_COUPLING).uniform(-1.0, 1.0, size=(E, ZONAL))
    if w.envelope:
        cpl = cpl * env[:, None]
    out["coupling"] = np.ascontiguousarray(cpl.astype(np.float32))
    out["env"] = env.astype(np.float32)
    if tiled_radial:
        out["radial_pool"] = radial_pool(w)
    else:
        out["radial"] = _rng(w.seed, _TAG_RADIAL).standard_normal(size=(E, SLOTS, C),
                                                                 dtype=np.float32)
    if with_grad:
        out["grad_out"] = _rng(w.seed, _TAG_GRAD).standard_normal(size=(N, ROWS, C), dtype=np.float32)
    return out


def custom(name: str, n_nodes: int, n_edges: int, channels: int, seed: int,
           dst_kind: str = "uniform", envelope: bool = False) -> Workload:
    """A workload outside the named five (edge cases, small parity sizes)."""
    return Workload(name, n_nodes, n_edges, channels, dst_kind, envelope, seed)


def fingerprint(arrays: dict) -> dict:
    """Short content hashes of every array, for recording alongside results."""
    fp = {}
    for k, v in arrays.items():
        if isinstance(v, np.ndarray):
            fp[k] = hashlib.blake2b(np.ascontiguousarray(v).view(np.uint8), digest_size=8).hexdigest()
    return fp


# Inputs past 2^31 elements.  Drawing billions of normals on the host takes
# minutes, so the radial tensor of such a workload is a seeded N(0,1) pool of
# prime length tiled over the flat (E, 3, C) array: element k is pool[k % P].
# Because P is prime, 2^32 is not a multiple of P, so an offset that wrapped
# at 32 bits would read a different pool entry.
RADIAL_POOL_LEN = 16777259   # prime, just above 2^24


def radial_pool(w: Workload, length: int = RADIAL_POOL_LEN) -> np.ndarray:
    """The seeded pool (float32, N(0,1)) a tiled radial tensor repeats."""
    return _rng(w.seed, _TAG_RADIAL).standard_normal(size=length, dtype=np.float32)


def tiled_radial_rows(pool: np.ndarray, edges: np.ndarray, channels: int) -> np.ndarray:
    """Rows radial[edges] (len(edges), 3, C) of the tiled radial tensor."""
    per_edge = SLOTS * channels
    k = np.asarray(edges, dtype=np.int64)[:, None] * per_edge + np.arange(per_edge, dtype=np.int64)
    return pool[k % pool.shape[0]].reshape(-1, SLOTS, channels)
