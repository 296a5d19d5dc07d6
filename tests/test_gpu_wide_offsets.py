"""Element offsets past 2^31 (needs a GPU, ~18 GB of HBM per case).

The radial input and grad_radial output hold E * 3 * C > 2^31 floats, so every
edge offset beyond e = 2^31 / (3 C) needs 64-bit address arithmetic; a 32-bit
wrap would read or write another edge's row.  Two shapes: C = 128 (the staged
forward and backward kernels) and C = 1024 (the largest channel count, generic
kernels).  The radial tensor tiles a seeded prime-length N(0,1) pool (element k
is pool[k mod P]) so that it can be built on the device in seconds; a wrapped
offset reads a different pool entry because 2^32 is not a multiple of P.

Checked against the oracle: the CSR in full (bitwise); the forward rows of
sampled nodes (bitwise), computed by the oracle on the sub-problem of exactly
those nodes' edges in increasing edge id (the per-node sums depend on nothing
else); grad_radial (bitwise) and grad_coupling (1e-6 + 1e-5 |ref|) of sampled
edges, weighted towards the last edges, where the offsets are largest.
"""
import sys

import numpy as np
import pytest
import torch

import edge_node_scatter_amd as zs
import oracle
import synthetic
from test_gpu_parity import _bits, check_grad_coupling

pytestmark = pytest.mark.gpu

CASES = [
    # label, N, E, C: E * 3 * C just above 2^31
    ("c128_5_6M_edges", 40000, 5600000, 128),
    ("c1024_700k_edges", 2000, 700000, 1024),
]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("label,N,E,C", CASES, ids=[c[0] for c in CASES])
def test_offsets_beyond_2g_elements(label, N, E, C):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert E * 3 * C > 2 ** 31
    dev = torch.device("cuda:0")
    zs.load()
    w = synthetic.custom(label, N, E, C, seed=7000 + C, envelope=True)
    x = synthetic.make_inputs(w, tiled_radial=True)
    pool = x["radial_pool"]
    say(f"[gpu] wide offsets {label}: N={N} E={E} C={C}, building inputs on the device")
    total = E * 3 * C
    reps = -(-total // pool.shape[0])
    rad = torch.from_numpy(pool).to(dev).repeat(reps)[:total].view(E, 3, C)
    cpl = torch.from_numpy(x["coupling"]).to(dev)
    g = torch.from_numpy(x["grad_out"]).to(dev)
    say(f"[gpu] wide offsets {label}: CSR, forward, backward")
    csr = zs.zs_build_csr(torch.from_numpy(x["dst"]).to(dev), N)
    out = zs.zs_forward(cpl, rad, csr)
    gc, gr = zs.zs_backward(g, cpl, rad, csr)
    torch.cuda.synchronize()

    rng = np.random.default_rng(17)
    first_wide = 2 ** 31 // (3 * C)               # first edge whose row starts past 2^31
    edges = np.unique(np.concatenate([
        [0, first_wide - 1, first_wide, first_wide + 1, E - 1],
        rng.integers(first_wide, E, 3000), rng.integers(0, E, 1000)]))
    nodes = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 14, replace=False)]))
    edges_t = torch.from_numpy(edges).to(dev)
    got = {"rowptr": csr.rowptr.cpu().numpy(), "perm": csr.perm.cpu().numpy(),
           "out": out[torch.from_numpy(nodes).to(dev)].cpu().numpy(),
           "row0": bool((out[:, 0] == 0).all().item()),
           "gc": gc[edges_t].cpu().numpy(), "gr": gr[edges_t].cpu().numpy()}
    del rad, cpl, g, csr, out, gc, gr, edges_t
    torch.cuda.empty_cache()
    say(f"[gpu] wide offsets {label}: comparing with the oracle")

    rowptr, perm = oracle.csr(x["dst"], N)
    assert np.array_equal(got["rowptr"], rowptr), f"{label}: rowptr"
    assert np.array_equal(got["perm"], perm), f"{label}: perm"
    assert got["row0"], f"{label}: row 0 must be +0"

    sub = np.flatnonzero(np.isin(x["dst"], nodes))          # increasing edge id
    sub_dst = np.searchsorted(nodes, x["dst"][sub])
    ref_out = oracle.forward(x["coupling"][sub], synthetic.tiled_radial_rows(pool, sub, C),
                             sub_dst, len(nodes))
    assert np.array_equal(_bits(got["out"]), _bits(ref_out)), f"{label}: sampled forward rows"

    ref_gc, ref_gr = oracle.backward(x["grad_out"], x["coupling"][edges],
                                     synthetic.tiled_radial_rows(pool, edges, C), x["dst"][edges])
    assert np.array_equal(_bits(got["gr"]), _bits(ref_gr)), f"{label}: sampled grad_radial"
    check_grad_coupling(got["gc"], ref_gc, f"{label}: sampled grad_coupling")
    say(f"[gpu] wide offsets {label}: parity ok")
