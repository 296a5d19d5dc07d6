"""Fused degree normalisation vs the oracle, through the C ABI (needs a GPU).

The GIE page ("What", third bullet) keeps an inverse-square-root degree
normalisation after the scatter, with its own envelope cotangent.  Bar, on the
same seeded inputs:
  * y, out, norm: bitwise (fixed edge order; correctly rounded sqrt and
    division on both sides);
  * grad_radial: bitwise;
  * grad_coupling and grad_env: |gpu - ref| <= 1e-6 + 1e-5 |ref| and at most
    one fp32 ulp apart (both round one fp64 sum of exact products);
  * grad_deg: equal to grad_env of every edge of the node, 0 for nodes
    without edges.
"""
import sys

import numpy as np
import pytest
import torch

import edge_node_scatter_amd as zs
import oracle
import synthetic
from cases import heavy_destinations

pytestmark = pytest.mark.gpu
ATOL, RTOL = 1e-6, 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    zs.load()
    return torch.device("cuda:0")


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _close(got, ref, what):
    inf = ~np.isfinite(ref)   # e.g. grad_env of a subnormal degree overflows fp32
    assert np.array_equal(_bits(got[inf]), _bits(ref[inf])), f"{what}: non-finite values"
    got, ref = got[~inf], ref[~inf]
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = ATOL + RTOL * np.abs(ref.astype(np.float64))
    assert np.all(diff <= tol), f"{what}: {np.count_nonzero(diff > tol)} outside tolerance"
    d = _bits(got) != _bits(ref)
    ulps = np.abs(_bits(got).astype(np.int64) - _bits(ref).astype(np.int64))
    assert np.all(ulps[d] <= 1), f"{what}: difference above one ulp"
    return int(np.count_nonzero(d))


def _bitwise(got, ref, what):
    nd = np.count_nonzero(_bits(got) != _bits(ref))
    assert nd == 0, f"{what}: {nd} bit differences"


def run_and_compare(x, n_nodes, dev, name, keep_out=True):
    say(f"[gpu] normalised {name}: N={n_nodes} E={len(x['dst'])} C={x['radial'].shape[2]}")
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "env",
                                                      "grad_out")}
    csr = zs.zs_build_csr(t["dst"], n_nodes)
    y, out, norm = zs.zs_forward_normalized(t["coupling"], t["radial"], t["env"], csr,
                                            keep_out=keep_out)
    if out is None:   # the backward needs the unnormalised scatter
        _, out, _ = zs.zs_forward_normalized(t["coupling"], t["radial"], t["env"], csr)
    gc, gr, ge, gd = zs.zs_backward_normalized(t["grad_out"], out, norm, t["coupling"],
                                               t["radial"], csr)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in dict(y=y, out=out, norm=norm, gc=gc, gr=gr, ge=ge,
                                                gd=gd).items()}
    ry, rout, rnorm = oracle.forward_norm(x["coupling"], x["radial"], x["env"], x["dst"],
                                          n_nodes)
    _bitwise(got["norm"], rnorm, f"{name}: norm")
    _bitwise(got["out"], rout, f"{name}: out")
    _bitwise(got["y"], ry, f"{name}: y")
    rgc, rgr, rge = oracle.backward_norm(x["grad_out"], rout, rnorm, x["coupling"], x["radial"],
                                         x["dst"])
    _bitwise(got["gr"], rgr, f"{name}: grad_radial")
    nc = _close(got["gc"], rgc, f"{name}: grad_coupling")
    ne = _close(got["ge"], rge, f"{name}: grad_env")
    # grad_deg is the per-node table grad_env is gathered from
    dst = x["dst"]
    assert np.array_equal(_bits(got["gd"][dst]), _bits(got["ge"])), f"{name}: grad_env gather"
    empty = np.bincount(dst, minlength=n_nodes) == 0
    assert np.all(_bits(got["gd"][empty]) == 0), f"{name}: grad_deg of empty nodes"
    assert np.all(_bits(got["norm"][empty]) == 0), f"{name}: norm of empty nodes"
    say(f"[gpu] normalised {name}: parity ok (ulp differences gc {nc}, genv {ne})")
    return got


@pytest.mark.parametrize("name", ["tiny", "n1000", "headline", "skewed"])
def test_normalized_workloads(dev, name):
    w = synthetic.WORKLOADS[name]
    x = synthetic.make_inputs(w)
    got = run_and_compare(x, w.n_nodes, dev, name)
    if name == "skewed":   # 64 vacuum nodes: deg 0 -> norm 0 -> y 0
        empty = np.bincount(x["dst"], minlength=w.n_nodes) == 0
        assert empty.sum() >= 64 and np.all(_bits(got["y"][empty]) == 0)


NORM_CASES = [
    # (label, N, E, C, dst kind) -- channel counts that take each kernel variant
    ("c4", 9, 300, 4, "uniform"),
    ("c8", 9, 300, 8, "uniform"),
    ("c24", 9, 300, 24, "uniform"),
    ("c48", 9, 300, 48, "uniform"),
    ("c56", 9, 300, 56, "uniform"),
    ("c100", 9, 300, 100, "uniform"),
    ("c20_scalar", 11, 500, 20, "uniform"),
    ("c36", 13, 700, 36, "uniform"),
    ("c64", 17, 900, 64, "uniform"),
    ("c96", 10, 800, 96, "uniform"),
    ("c33_scalar", 8, 400, 33, "uniform"),
    ("one_edge", 5, 1, 32, "uniform"),
    ("hub", 3, 5000, 32, "uniform"),
    ("grid_stride_c8", 1_200_000, 2_400_000, 8, "uniform"),   # more nodes than one grid holds
    ("n2500_batch8", 2500, 40000, 32, "uniform"),
    ("staged_c48", 1300, 30000, 48, "uniform"),     # one-wavefront-per-tile forward, 6 ch/lane
    ("slot_b8", 1500, 30000, 32, "uniform"),        # slot-split forward, 8-edge batches
    # heavy nodes (several thousand edges) beside light ones, envelope sums included
    ("split_c32", 3000, 200000, 32, "heavy"),
    ("split_c16", 2600, 150000, 16, "heavy"),
    ("split_c8", 2600, 120000, 8, "heavy"),
    ("heavy_b4_c32", 4096, 300000, 32, "heavy"),    # 4-edge batches, heavy nodes 8-edge
    ("heavy_b4_c8", 4500, 200000, 8, "heavy"),
    ("split_grid_stride_c8", 1_100_000, 2_300_000, 8, "heavy"),
]


@pytest.mark.parametrize("label,N,E,C,kind", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_normalized_shapes(dev, label, N, E, C, kind):
    w = synthetic.custom(label, N, E, C, seed=9100 + E,
                         dst_kind="uniform" if kind == "heavy" else kind, envelope=True)
    x = synthetic.make_inputs(w)
    if kind == "heavy":
        x["dst"] = heavy_destinations(E, N, seed=E + C)
    run_and_compare(x, N, dev, label)


def test_normalized_large(dev):
    """The 16384-node, C = 64 frame (E = 2.6M) through the normalised pair,
    compared with the oracle in full."""
    w = synthetic.WORKLOADS["large"]
    run_and_compare(synthetic.make_inputs(w), w.n_nodes, dev, "large")


def test_normalized_without_out(dev):
    w = synthetic.WORKLOADS["n1000"]
    run_and_compare(synthetic.make_inputs(w), w.n_nodes, dev, "n1000_no_out", keep_out=False)


def test_normalized_zero_and_tiny_envelopes(dev):
    """Envelopes of exactly 0 (edges at the cutoff) and subnormal ones."""
    w = synthetic.custom("env_edge", 12, 600, 32, seed=9301, envelope=True)
    x = synthetic.make_inputs(w)
    env = x["env"].copy()
    env[x["dst"] == 3] = 0.0                       # node 3: edges but zero degree
    env[x["dst"] == 5] = np.float32(1e-40)         # node 5: subnormal degree
    x["env"] = env
    got = run_and_compare(x, w.n_nodes, dev, "env_edge")
    # norm 0 times a negative sum is -0 on both sides (the bitwise check above)
    assert got["norm"][3] == 0.0 and np.all(got["y"][3] == 0.0)
    assert np.isfinite(got["norm"][5]) and got["norm"][5] > 1e18


def test_normalized_no_edges(dev):
    N, C = 6, 32
    dst = torch.zeros(0, dtype=torch.int64, device=dev)
    csr = zs.zs_build_csr(dst, N)
    cpl = torch.zeros((0, 15), device=dev)
    rad = torch.zeros((0, 3, C), device=dev)
    env = torch.zeros(0, device=dev)
    y, out, norm = zs.zs_forward_normalized(cpl, rad, env, csr)
    gy = torch.randn((N, 16, C), device=dev)
    gc, gr, ge, gd = zs.zs_backward_normalized(gy, out, norm, cpl, rad, csr)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0 and torch.count_nonzero(out) == 0
    assert torch.count_nonzero(norm) == 0 and torch.count_nonzero(gd) == 0
    assert gc.shape == (0, 15) and gr.shape == (0, 3, C) and ge.shape == (0,)


def test_normalized_deterministic(dev):
    w = synthetic.WORKLOADS["headline"]
    x = synthetic.make_inputs(w)
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "env",
                                                      "grad_out")}
    csr = zs.zs_build_csr(t["dst"], w.n_nodes)
    say("[gpu] normalised determinism: headline x5")
    first = None
    for _ in range(5):
        y, out, norm = zs.zs_forward_normalized(t["coupling"], t["radial"], t["env"], csr)
        grads = zs.zs_backward_normalized(t["grad_out"], out, norm, t["coupling"], t["radial"],
                                          csr)
        cur = [a.cpu().numpy().view(np.uint8) for a in (y, out, norm, *grads)]
        if first is None:
            first = cur
        for a, b in zip(first, cur):
            assert np.array_equal(a, b)


def test_normalized_autograd(dev):
    w = synthetic.custom("autograd_norm", 40, 3000, 32, seed=9401, envelope=True)
    x = synthetic.make_inputs(w)
    dst = torch.from_numpy(x["dst"]).to(dev)
    csr = zs.zs_build_csr(dst, w.n_nodes)
    cpl = torch.from_numpy(x["coupling"]).to(dev).requires_grad_(True)
    rad = torch.from_numpy(x["radial"]).to(dev).requires_grad_(True)
    env = torch.from_numpy(x["env"]).to(dev).requires_grad_(True)
    y = zs.gie_zonal_scatter_normalized(cpl, rad, env, csr)
    assert isinstance(y, torch.Tensor) and y.requires_grad
    gy = torch.from_numpy(x["grad_out"]).to(dev)
    y.backward(gy)
    torch.cuda.synchronize()
    ry, rout, rnorm = oracle.forward_norm(x["coupling"], x["radial"], x["env"], x["dst"],
                                          w.n_nodes)
    _bitwise(y.detach().cpu().numpy(), ry, "autograd: y")
    rgc, rgr, rge = oracle.backward_norm(x["grad_out"], rout, rnorm, x["coupling"], x["radial"],
                                         x["dst"])
    _bitwise(rad.grad.cpu().numpy(), rgr, "autograd: grad_radial")
    _close(cpl.grad.cpu().numpy(), rgc, "autograd: grad_coupling")
    _close(env.grad.cpu().numpy(), rge, "autograd: grad_env")


def test_normalized_backward_unaligned_out(dev):
    """out at a 4-byte (not 16-byte) offset: the degree gradient then comes from
    the separate per-node kernel instead of the backward's row staging."""
    w = synthetic.custom("unaligned_out", 50, 4000, 32, seed=9501, envelope=True)
    x = synthetic.make_inputs(w)
    N, C = w.n_nodes, w.channels
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "env",
                                                      "grad_out")}
    csr = zs.zs_build_csr(t["dst"], N)
    y, out, norm = zs.zs_forward_normalized(t["coupling"], t["radial"], t["env"], csr)
    storage = torch.empty(N * 16 * C + 1, device=dev)
    out_off = storage[1:].view(N, 16, C)
    out_off.copy_(out)
    assert out_off.data_ptr() % 16 == 4
    say("[gpu] normalised backward with a 4-byte-offset out")
    gc, gr, ge, gd = zs.zs_backward_normalized(t["grad_out"], out_off, norm, t["coupling"],
                                               t["radial"], csr)
    torch.cuda.synchronize()
    ry, rout, rnorm = oracle.forward_norm(x["coupling"], x["radial"], x["env"], x["dst"], N)
    rgc, rgr, rge = oracle.backward_norm(x["grad_out"], rout, rnorm, x["coupling"], x["radial"],
                                         x["dst"])
    _bitwise(gr.cpu().numpy(), rgr, "unaligned out: grad_radial")
    _close(gc.cpu().numpy(), rgc, "unaligned out: grad_coupling")
    _close(ge.cpu().numpy(), rge, "unaligned out: grad_env")
    assert np.array_equal(_bits(gd.cpu().numpy()[x["dst"]]), _bits(ge.cpu().numpy()))
