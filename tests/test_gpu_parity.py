"""HIP path vs the oracle, element by element, through the C ABI (needs a GPU).

Bar (all configurations, same seeded inputs on both sides):
  * CSR rowptr / perm / dst32: bitwise (integer work);
  * forward out: bitwise (fixed edge order, separate fp32 multiply and add);
  * grad_radial: bitwise (fixed row order);
  * grad_coupling: |gpu - ref| <= 1e-6 + 1e-5 |ref| elementwise (the stated
    fp32 tolerance); both sides sum exact products in fp64 and round once, so
    at most a few near-ties may differ, by one fp32 ulp.
Every workload is compared in full, the large one (E = 2.6M, C = 64) too; it
also checks the oracle's sampled entry points (used where the full oracle would
not fit, as for offsets past 2^31) and size-independent properties.
The node schedule the CSR build also returns (the order in which the forward
hands out nodes, not a result of the method) is checked against its
definition in include/zs.h: per-bucket degree ranks laid out rank-major, the
identity above 16384 nodes.
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


def run_gpu(x, dev, n_nodes):
    dst = torch.from_numpy(x["dst"]).to(dev)
    cpl = torch.from_numpy(x["coupling"]).to(dev)
    rad = torch.from_numpy(x["radial"]).to(dev)
    g = torch.from_numpy(x["grad_out"]).to(dev)
    csr = zs.zs_build_csr(dst, n_nodes)
    out = zs.zs_forward(cpl, rad, csr)
    gc, gr = zs.zs_backward(g, cpl, rad, csr)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in
            dict(rowptr=csr.rowptr, perm=csr.perm, dst32=csr.dst32, order=csr.order, out=out,
                 gc=gc, gr=gr).items()}


def expected_order(rowptr):
    """The node schedule as include/zs.h defines it: buckets of B consecutive
    nodes (B the smallest power of two >= N / 256), each ranked by decreasing
    degree (ties by node id), rank r of full bucket b at r*F + (b + r) mod F
    (F full buckets), the partial bucket's ranks after them; identity when
    B > 64."""
    n = len(rowptr) - 1
    bn = 1
    while bn * 256 < n:
        bn *= 2
    if bn > 64:
        return np.arange(n, dtype=np.int32)
    deg = np.diff(rowptr.astype(np.int64))
    nf = n // bn
    order = np.full(n, -1, dtype=np.int64)
    for b in range(-(-n // bn)):
        nodes = np.arange(b * bn, min(n, (b + 1) * bn))
        ranked = nodes[np.lexsort((nodes, -deg[nodes]))]
        for r, node in enumerate(ranked):
            order[r * nf + (b + r) % nf if b < nf else nf * bn + r] = node
    assert np.array_equal(np.sort(order), np.arange(n))
    return order.astype(np.int32)


def check_order(order, rowptr, name):
    assert np.array_equal(order, expected_order(rowptr)), \
        f"{name}: node order, {np.count_nonzero(order != expected_order(rowptr))} entries differ"


def check_grad_coupling(got, ref, what):
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = ATOL + RTOL * np.abs(ref.astype(np.float64))
    assert np.all(diff <= tol), f"{what}: {np.count_nonzero(diff > tol)} outside tolerance"
    nbits = np.count_nonzero(_bits(got) != _bits(ref))
    ulps = np.abs(_bits(got).astype(np.int64) - _bits(ref).astype(np.int64))
    assert nbits <= max(4, got.size // 100000), f"{what}: {nbits} bit differences"
    assert np.all(ulps[_bits(got) != _bits(ref)] <= 1), f"{what}: difference above one ulp"
    return nbits


def compare_full(x, res, n_nodes, name):
    rowptr, perm = oracle.csr(x["dst"], n_nodes)
    assert np.array_equal(res["rowptr"], rowptr), f"{name}: rowptr"
    assert np.array_equal(res["perm"], perm), f"{name}: perm"
    assert np.array_equal(res["dst32"], x["dst"].astype(np.int32)), f"{name}: dst32"
    if "order" in res:
        check_order(res["order"], rowptr, name)
    out = oracle.forward(x["coupling"], x["radial"], x["dst"], n_nodes)
    assert np.array_equal(_bits(res["out"]), _bits(out)), \
        f"{name}: forward, {np.count_nonzero(_bits(res['out']) != _bits(out))} bit differences"
    gc, gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    assert np.array_equal(_bits(res["gr"]), _bits(gr)), \
        f"{name}: grad_radial, {np.count_nonzero(_bits(res['gr']) != _bits(gr))} bit differences"
    return check_grad_coupling(res["gc"], gc, f"{name}: grad_coupling")


@pytest.mark.parametrize("name", ["tiny", "n1000", "headline", "skewed", "headline_grouped",
                                  "headline_uniform"])
def test_workload_full(dev, name):
    w = synthetic.WORKLOADS[name]
    x = synthetic.make_inputs(w)
    say(f"[gpu] workload {name}: N={w.n_nodes} E={w.n_edges} C={w.channels}")
    res = run_gpu(x, dev, w.n_nodes)
    nbits = compare_full(x, res, w.n_nodes, name)
    say(f"[gpu] workload {name}: parity ok, grad_coupling bit differences {nbits}")


def test_workload_large(dev):
    """The 16384-node, C = 64 frame compared with the oracle element by element
    (the sequential oracle takes a few seconds here), then the sampled oracle
    entry points against the same GPU results, then properties that hold at
    any size."""
    w = synthetic.WORKLOADS["large"]
    x = synthetic.make_inputs(w)
    say(f"[gpu] workload large: N={w.n_nodes} E={w.n_edges} C={w.channels}")
    res = run_gpu(x, dev, w.n_nodes)
    compare_full(x, res, w.n_nodes, "large")
    rng = np.random.default_rng(1)
    nodes = np.concatenate([[0, w.n_nodes - 1], rng.choice(w.n_nodes, 62, replace=False)])
    ref_rows = oracle.forward_nodes(x["coupling"], x["radial"], x["dst"], w.n_nodes, nodes)
    assert np.array_equal(_bits(res["out"][nodes]), _bits(ref_rows)), "large: sampled forward rows"
    edges = np.concatenate([[0, w.n_edges - 1], rng.choice(w.n_edges, 20000, replace=False)])
    gc, gr = oracle.backward_edges(x["grad_out"], x["coupling"], x["radial"], x["dst"], edges)
    assert np.array_equal(_bits(res["gr"][edges]), _bits(gr)), "large: sampled grad_radial"
    check_grad_coupling(res["gc"][edges], gc, "large: sampled grad_coupling")
    # size-independent properties over the whole output
    assert np.all(_bits(res["out"][:, 0]) == 0), "row 0 must be +0"
    deg = np.bincount(x["dst"], minlength=w.n_nodes)
    for r in (1, 5, 12):
        s = 0 if r < 4 else (1 if r < 9 else 2)
        tot = x["coupling"][:, r - 1].astype(np.float64) @ x["radial"][:, s, :].astype(np.float64)
        got = res["out"][:, r, :].astype(np.float64).sum(axis=0)
        scale = np.abs(x["coupling"][:, r - 1]).astype(np.float64) @ \
            np.abs(x["radial"][:, s, :]).astype(np.float64)
        assert np.all(np.abs(got - tot) <= (deg.max() + 2) * 2.0 ** -24 * scale + 1e-30), \
            f"large: total message row {r}"


def test_deterministic_headline(dev):
    w = synthetic.WORKLOADS["headline"]
    x = synthetic.make_inputs(w)
    say("[gpu] determinism: headline x10")
    first = run_gpu(x, dev, w.n_nodes)
    for _ in range(9):
        again = run_gpu(x, dev, w.n_nodes)
        for k in first:
            assert np.array_equal(first[k].view(np.uint8), again[k].view(np.uint8)), k


EDGE_CASES = [
    # (label, N, E, C, dst kind)
    ("one_edge", 5, 1, 32, "uniform"),
    ("one_node", 1, 3001, 32, "uniform"),
    ("e37", 9, 37, 32, "uniform"),
    ("e63", 7, 63, 16, "uniform"),
    ("e64", 7, 64, 8, "uniform"),
    ("e65", 7, 65, 4, "uniform"),
    ("tile_2047", 40, 2047, 32, "uniform"),
    ("tile_2048", 40, 2048, 32, "uniform"),
    ("tile_2049", 40, 2049, 32, "uniform"),
    ("e8193", 300, 8193, 32, "uniform"),
    ("mostly_empty", 5000, 300, 32, "uniform"),
    ("c1", 17, 500, 1, "uniform"),
    ("c2", 17, 500, 2, "uniform"),
    ("c3", 17, 500, 3, "uniform"),
    ("c5", 17, 500, 5, "uniform"),
    ("c4", 17, 500, 4, "uniform"),
    ("c12", 17, 500, 12, "uniform"),
    ("c16", 17, 500, 16, "uniform"),
    ("c24", 17, 500, 24, "uniform"),
    ("c28", 17, 500, 28, "uniform"),
    ("c31", 17, 500, 31, "uniform"),
    ("c33", 17, 500, 33, "uniform"),
    ("c36", 17, 500, 36, "uniform"),
    ("c40_pages", 33, 777, 40, "uniform"),
    ("c44", 17, 500, 44, "uniform"),
    ("c48", 17, 500, 48, "uniform"),
    ("c52", 17, 500, 52, "uniform"),
    ("c56", 17, 500, 56, "uniform"),
    ("c60", 17, 500, 60, "uniform"),
    ("c63", 17, 500, 63, "uniform"),
    ("c64", 17, 500, 64, "uniform"),
    ("c65", 17, 500, 65, "uniform"),
    ("c68", 17, 500, 68, "uniform"),
    ("c96", 17, 500, 96, "uniform"),
    ("c100", 17, 500, 100, "uniform"),
    ("c128", 17, 700, 128, "uniform"),
    ("c260", 9, 300, 260, "uniform"),
    ("c1024", 3, 70, 1024, "uniform"),
    ("skew_small", 200, 9000, 32, "skewed_small"),
    ("nodes_20000", 20000, 40000, 8, "uniform"),      # many buckets; 4-edge forward batches
    ("nodes_3000", 3000, 90000, 32, "uniform"),       # 8-edge forward batches (2048..4095 waves)
    # Frames with fewer wavefronts go to the slot-split forward (16-edge
    # batches below 1280 wavefronts, 8-edge below 2048 at <= 4 channels per
    # lane); these keep the one-wavefront-per-tile forward covered at every
    # channel width, and the slot kernel at its 8-edge batches.
    ("staged_c16", 2100, 40000, 16, "uniform"),
    ("staged_c24", 2100, 40000, 24, "uniform"),
    ("staged_c40", 1300, 40000, 40, "uniform"),
    ("staged_c48", 1300, 40000, 48, "uniform"),
    ("staged_c56", 1300, 40000, 56, "uniform"),
    ("staged_c64", 1300, 40000, 64, "uniform"),
    ("staged_c100", 1300, 30000, 100, "uniform"),     # two 64-channel tiles, the second partial
    ("slot_b8_c32", 1500, 40000, 32, "uniform"),
    ("slot_b8_c12", 1900, 40000, 12, "uniform"),
    # More nodes than one launch's grid holds (2^20 forward workgroups, 2^20
    # backward work items = 2^18 nodes): the kernels' grid-stride node loops.
    ("grid_stride_c8", 1_200_000, 2_400_000, 8, "uniform"),
    ("grid_stride_c16", 1_100_000, 1_500_000, 16, "uniform"),
    # Heavy nodes (degree at least 1.5x the mean, up to several thousand
    # edges) beside light ones in launches of the one-wavefront-per-node
    # forward and the split-item backward, at each channel width up to 4 per
    # lane, and on both sides of the grid-stride pass.
    ("split_c32", 3000, 200000, 32, "heavy"),
    ("split_c28", 2600, 150000, 28, "heavy"),
    ("split_c24", 2600, 150000, 24, "heavy"),
    ("split_c16", 2600, 150000, 16, "heavy"),
    ("split_c12", 2600, 120000, 12, "heavy"),
    ("split_c8", 2600, 120000, 8, "heavy"),
    ("split_c4", 2600, 100000, 4, "heavy"),
    ("split_grid_stride_c8", 1_100_000, 2_300_000, 8, "heavy"),
    # Launches of at least 4096 wavefronts take 4-edge batches, and nodes
    # above 5/4 of the mean degree 8-edge ones (with the node schedule putting
    # them first): both paths at each channel width up to 4 per lane.
    ("heavy_b4_c32", 4096, 300000, 32, "heavy"),
    ("heavy_b4_c24", 4096, 250000, 24, "heavy"),
    ("heavy_b4_c16", 4200, 250000, 16, "heavy"),
    ("heavy_b4_c8", 4500, 200000, 8, "heavy"),
    ("heavy_b4_c4", 5000, 150000, 4, "heavy"),
    ("heavy_nodes_20000_c8", 20000, 400000, 8, "heavy"),   # identity schedule above 16384 nodes
    ("sched_partial_c8", 3333, 120000, 8, "heavy"),     # 16-node buckets, a partial one of 5
]



@pytest.mark.parametrize("label,N,E,C,kind", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_cases(dev, label, N, E, C, kind):
    w = synthetic.custom(label, N, E, C, seed=1000 + len(label) * 7 + C, envelope=True)
    x = synthetic.make_inputs(w)
    if kind == "skewed_small":
        rng = np.random.default_rng(5)
        x["dst"] = np.where(rng.random(E) < 0.7, rng.integers(0, 10, E), rng.integers(0, N, E))
    elif kind == "heavy":
        x["dst"] = heavy_destinations(E, N, seed=len(label) + C)
        deg = np.bincount(x["dst"], minlength=N)
        hmin = max(64, -(-3 * E // (2 * N)))
        assert np.count_nonzero(deg >= hmin) >= 3 and deg[N - 1] >= hmin
    say(f"[gpu] edge case {label}: N={N} E={E} C={C}")
    res = run_gpu(x, dev, N)
    compare_full(x, res, N, label)


def test_all_edges_one_node(dev):
    N, E, C = 50, 20000, 32
    w = synthetic.custom("hub", N, E, C, seed=77)
    x = synthetic.make_inputs(w)
    x["dst"] = np.full(E, 7, dtype=np.int64)
    say("[gpu] hub node: all 20000 edges on node 7")
    res = run_gpu(x, dev, N)
    compare_full(x, res, N, "hub")


def test_no_edges(dev):
    say("[gpu] E = 0")
    N, C = 6, 32
    dst = torch.zeros(0, dtype=torch.int64, device=dev)
    cpl = torch.zeros((0, 15), device=dev)
    rad = torch.zeros((0, 3, C), device=dev)
    csr = zs.zs_build_csr(dst, N)
    out = zs.zs_forward(cpl, rad, csr, out=torch.full((N, 16, C), float("nan"), device=dev))
    gc, gr = zs.zs_backward(torch.ones((N, 16, C), device=dev), cpl, rad, csr)
    torch.cuda.synchronize()
    assert torch.equal(csr.rowptr.cpu(), torch.zeros(N + 1, dtype=torch.int32))
    assert torch.equal(csr.order.cpu(), torch.arange(N, dtype=torch.int32))
    assert np.all(_bits(out.cpu().numpy()) == 0)
    assert gc.shape == (0, 15) and gr.shape == (0, 3, C)


def test_two_streams_at_once(dev):
    """Two frames in flight at the same time on two streams, their launches
    interleaved: every call works only on its own stream and buffers, so each
    frame matches the oracle as if it ran alone."""
    frames = [(synthetic.custom("stream_a", 300, 40000, 32, seed=71), 300),
              (synthetic.custom("stream_b", 211, 31000, 24, seed=72), 211)]
    say("[gpu] two streams: N=300 E=40000 C=32 and N=211 E=31000 C=24")
    xs = [synthetic.make_inputs(w) for w, _ in frames]
    ts = [{k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "grad_out")}
          for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    state = [dict() for _ in frames]
    for phase in ("build", "forward", "backward"):
        for (w, N), s, t, st in zip(frames, streams, ts, state):
            with torch.cuda.stream(s):
                if phase == "build":
                    st["flag"] = torch.zeros(1, dtype=torch.int32, device=dev)
                    st["csr"] = zs.zs_build_csr(t["dst"], N, bad_flag=st["flag"])
                elif phase == "forward":
                    st["out"] = zs.zs_forward(t["coupling"], t["radial"], st["csr"])
                else:
                    st["gc"], st["gr"] = zs.zs_backward(t["grad_out"], t["coupling"],
                                                        t["radial"], st["csr"])
    torch.cuda.synchronize()
    for (w, N), x, st in zip(frames, xs, state):
        assert int(st["flag"].item()) == 0
        csr = st["csr"]
        res = {k: v.cpu().numpy() for k, v in dict(
            rowptr=csr.rowptr, perm=csr.perm, dst32=csr.dst32, out=st["out"], gc=st["gc"],
            gr=st["gr"]).items()}
        compare_full(x, res, N, w.name)


def test_wrong_buffers_rejected_before_launch(dev):
    """Output buffers and CSR arrays of the wrong size are refused by the
    binding, and the buffers they would have overrun are left untouched."""
    say("[gpu] wrong-sized buffers")
    N, E, C = 9, 300, 32
    w = synthetic.custom("wrongbuf", N, E, C, seed=5)
    x = synthetic.make_inputs(w)
    cpl = torch.from_numpy(x["coupling"]).to(dev)
    rad = torch.from_numpy(x["radial"]).to(dev)
    g = torch.from_numpy(x["grad_out"]).to(dev)
    csr = zs.zs_build_csr(torch.from_numpy(x["dst"]).to(dev), N)
    small = torch.full((N - 1, 16, C), float("nan"), device=dev)
    with pytest.raises(ValueError):
        zs.zs_forward(cpl, rad, csr, out=small)
    with pytest.raises(ValueError):
        zs.zs_backward(g, cpl, rad, csr, grad_radial=torch.empty((E - 1, 3, C), device=dev))
    short = csr._replace(rowptr=csr.rowptr[:N])
    with pytest.raises(ValueError):
        zs.zs_forward(cpl, rad, short)
    with pytest.raises(ValueError):
        zs.zs_build_csr(torch.from_numpy(x["dst"]).to(dev), N, out=csr._replace(perm=csr.perm[1:]))
    torch.cuda.synchronize()
    assert torch.isnan(small).all()


def test_bad_destination_rejected(dev):
    N, E = 10, 5000
    for bad in (N, -1, 1 << 40):
        say(f"[gpu] bad destination {bad}")
        d = torch.zeros(E, dtype=torch.int64)
        d[E // 3] = bad
        with pytest.raises(zs.ZsError) as ei:
            zs.zs_build_csr(d.to(dev), N)
        assert ei.value.status == -3


CSR_ONLY_CASES = [
    # (label, N, E): node counts around the bucket-size limits of the CSR build
    ("n_4194304_lds_nodes", 1 << 22, 100000),        # 2048-node buckets, LDS tables
    ("n_4194305_global_nodes", (1 << 22) + 1, 100000),  # 4096-node buckets, global tables
    ("n_5000000_sparse", 5_000_000, 30000),
    ("n_65536_many_buckets", 1 << 16, 700000),
    ("n_1_all_one_node", 1, 100000),
]


@pytest.mark.parametrize("label,N,E", CSR_ONLY_CASES, ids=[c[0] for c in CSR_ONLY_CASES])
def test_csr_only_node_counts(dev, label, N, E):
    say(f"[gpu] csr {label}: N={N} E={E}")
    rng = np.random.default_rng(N % 1000 + E)
    dst = rng.integers(0, N, E, dtype=np.int64)
    csr = zs.zs_build_csr(torch.from_numpy(dst).to(dev), N)
    torch.cuda.synchronize()
    rowptr, perm = oracle.csr(dst, N)
    assert np.array_equal(csr.rowptr.cpu().numpy(), rowptr), f"{label}: rowptr"
    assert np.array_equal(csr.perm.cpu().numpy(), perm), f"{label}: perm"
    assert np.array_equal(csr.dst32.cpu().numpy(), dst.astype(np.int32)), f"{label}: dst32"
    check_order(csr.order.cpu().numpy(), rowptr, label)


def test_guard_regions_and_unaligned(dev):
    """Outputs inside NaN-poisoned buffers: nothing outside them is written and
    nothing past the inputs is read; a one-float offset takes the scalar path."""
    E, N, C = 777, 33, 40                      # the pages' non-power-of-two case
    w = synthetic.custom("guard", N, E, C, seed=4040)
    x = synthetic.make_inputs(w)
    ref_out = oracle.forward(x["coupling"], x["radial"], x["dst"], N)
    ref_gc, ref_gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    for off in (0, 1):
        say(f"[gpu] guard regions, offset {off}")
        G = 4096

        def poisoned(arr):
            buf = torch.full((off + arr.size + G,), float("nan"), device=dev)
            buf[off:off + arr.size] = torch.from_numpy(arr.ravel()).to(dev)
            return buf, buf[off:off + arr.size].view(arr.shape)

        _, cpl = poisoned(x["coupling"])
        _, rad = poisoned(x["radial"])
        _, g = poisoned(x["grad_out"])
        csr = zs.zs_build_csr(torch.from_numpy(x["dst"]).to(dev), N)
        obuf = torch.full((off + N * 16 * C + G,), float("nan"), device=dev)
        out = obuf[off:off + N * 16 * C].view(N, 16, C)
        gcbuf = torch.full((off + E * 15 + G,), float("nan"), device=dev)
        grbuf = torch.full((off + E * 3 * C + G,), float("nan"), device=dev)
        gc = gcbuf[off:off + E * 15].view(E, 15)
        gr = grbuf[off:off + E * 3 * C].view(E, 3, C)
        zs.zs_forward(cpl, rad, csr, out=out)
        zs.zs_backward(g, cpl, rad, csr, grad_coupling=gc, grad_radial=gr)
        torch.cuda.synchronize()
        for buf, n in ((obuf, N * 16 * C), (gcbuf, E * 15), (grbuf, E * 3 * C)):
            b = buf.cpu().numpy()
            assert np.all(np.isnan(b[:off])) and np.all(np.isnan(b[off + n:])), "write outside output"
        assert np.array_equal(_bits(out.cpu().numpy()), _bits(ref_out))
        assert np.array_equal(_bits(gr.cpu().numpy()), _bits(ref_gr))
        check_grad_coupling(gc.cpu().numpy(), ref_gc, "guard grad_coupling")


def test_inputs_not_modified(dev):
    w = synthetic.custom("immut", 100, 5000, 32, seed=9)
    x = synthetic.make_inputs(w)
    say("[gpu] inputs unchanged")
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "grad_out")}
    before = {k: v.clone() for k, v in t.items()}
    csr = zs.zs_build_csr(t["dst"], 100)
    zs.zs_forward(t["coupling"], t["radial"], csr)
    zs.zs_backward(t["grad_out"], t["coupling"], t["radial"], csr)
    torch.cuda.synchronize()
    for k in t:
        assert torch.equal(t[k], before[k]), k


def test_autograd_function_sliced_radial(dev):
    """The autograd wrapper (contiguous and sliced-view radial) against the oracle."""
    w = synthetic.custom("autograd", 40, 3000, 32, seed=31)
    x = synthetic.make_inputs(w)
    say("[gpu] autograd wrapper")
    csr = zs.zs_build_csr(torch.from_numpy(x["dst"]).to(dev), 40)
    ref_out = oracle.forward(x["coupling"], x["radial"], x["dst"], 40)
    ref_gc, ref_gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    wide = torch.randn((3000, 5, 32), device=dev)
    wide[:, 1:4] = torch.from_numpy(x["radial"]).to(dev)
    for rad in (torch.from_numpy(x["radial"]).to(dev), wide[:, 1:4]):
        cpl = torch.from_numpy(x["coupling"]).to(dev).requires_grad_(True)
        rad = rad.detach().requires_grad_(True)
        out = zs.gie_zonal_scatter(cpl, rad, csr)
        out.backward(torch.from_numpy(x["grad_out"]).to(dev))
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out.detach().cpu().numpy()), _bits(ref_out))
        assert np.array_equal(_bits(rad.grad.cpu().numpy()), _bits(ref_gr))
        check_grad_coupling(cpl.grad.cpu().numpy(), ref_gc, "autograd grad_coupling")


STRIDED_CASES = [
    # (label, N, E, C, radial slab width (slots in the wider tensor), radial slot offset, band)
    ("sliced_radial_c32", 64, 3000, 32, 5, 1, False),
    ("band_coupling_c32", 64, 3000, 32, 3, 0, True),
    ("both_c32", 300, 20000, 32, 4, 1, True),
    ("both_c64", 50, 5000, 64, 6, 2, True),
    ("sliced_c40", 33, 777, 40, 5, 1, True),
    ("odd_stride_c33", 20, 900, 33, 4, 1, True),          # strides not multiples of 4
    ("sliced_c36", 20, 900, 36, 4, 1, False),
]


def _strided_inputs(x, dev, slab, s0, band):
    """Views of wider device tensors that hold the workload's inputs."""
    E, C = x["radial"].shape[0], x["radial"].shape[2]
    rng = np.random.default_rng(E + C)
    wide = torch.from_numpy(rng.standard_normal((E, slab, C + (1 if C % 2 else 0)),
                                                dtype=np.float32)).to(dev)
    wide[:, s0:s0 + 3, :C] = torch.from_numpy(x["radial"]).to(dev)
    rad = wide[:, s0:s0 + 3, :C]
    if band:
        b = torch.from_numpy(rng.standard_normal((E, 46), dtype=np.float32)).to(dev)
        cpl = zs.coupling_from_band(b)
        cpl.copy_(torch.from_numpy(x["coupling"]).to(dev))
    else:
        cpl = torch.from_numpy(x["coupling"]).to(dev)
    return cpl, rad


@pytest.mark.parametrize("label,N,E,C,slab,s0,band", STRIDED_CASES,
                         ids=[c[0] for c in STRIDED_CASES])
def test_strided_views(dev, label, N, E, C, slab, s0, band):
    """Sliced radial features and the coupling inside a packed (E, 46) band are
    read in place and give the oracle's results for the contiguous inputs."""
    w = synthetic.custom(label, N, E, C, seed=5000 + E + C, envelope=True)
    x = synthetic.make_inputs(w)
    say(f"[gpu] strided views {label}: N={N} E={E} C={C}")
    cpl, rad = _strided_inputs(x, dev, slab, s0, band)
    assert not rad.is_contiguous() or not cpl.is_contiguous()
    csr = zs.zs_build_csr(torch.from_numpy(x["dst"]).to(dev), N)
    out = zs.zs_forward(cpl, rad, csr)
    gc, gr = zs.zs_backward(torch.from_numpy(x["grad_out"]).to(dev), cpl, rad, csr)
    torch.cuda.synchronize()
    ref_out = oracle.forward(x["coupling"], x["radial"], x["dst"], N)
    ref_gc, ref_gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(ref_out)), f"{label}: forward"
    assert np.array_equal(_bits(gr.cpu().numpy()), _bits(ref_gr)), f"{label}: grad_radial"
    check_grad_coupling(gc.cpu().numpy(), ref_gc, f"{label}: grad_coupling")


@pytest.mark.parametrize("label,N,E,C", [("bcast_c32", 50, 3000, 32), ("bcast_c12", 17, 777, 12)])
def test_broadcast_views(dev, label, N, E, C):
    """Zero strides (the header allows them: inputs are only read): the
    coupling and radial rows broadcast to every edge, and a radial view whose
    three slots alias one row.  Results equal the oracle on materialised
    copies of the same views."""
    w = synthetic.custom(label, N, E, C, seed=6100 + E + C)
    x = synthetic.make_inputs(w)
    say(f"[gpu] broadcast views {label}: N={N} E={E} C={C}")
    dst = torch.from_numpy(x["dst"]).to(dev)
    csr = zs.zs_build_csr(dst, N)
    g = torch.from_numpy(x["grad_out"]).to(dev)
    row_c = torch.from_numpy(x["coupling"][:1].copy()).to(dev)          # (1, 15)
    row_r = torch.from_numpy(x["radial"][:1].copy()).to(dev)            # (1, 3, C)
    slot_r = torch.from_numpy(x["radial"][:, :1].copy()).to(dev)        # (E, 1, C)
    cases = {
        "both rows broadcast": (row_c.expand(E, 15), row_r.expand(E, 3, C)),
        "radial slots aliased": (torch.from_numpy(x["coupling"]).to(dev), slot_r.expand(E, 3, C)),
    }
    for what, (cpl, rad) in cases.items():
        assert cpl.stride(0) == 0 or rad.stride(1) == 0
        out = zs.zs_forward(cpl, rad, csr)
        gc, gr = zs.zs_backward(g, cpl, rad, csr)
        torch.cuda.synchronize()
        c_np = np.ascontiguousarray(cpl.cpu().numpy())
        r_np = np.ascontiguousarray(rad.cpu().numpy())
        ref_out = oracle.forward(c_np, r_np, x["dst"], N)
        ref_gc, ref_gr = oracle.backward(x["grad_out"], c_np, r_np, x["dst"])
        assert np.array_equal(_bits(out.cpu().numpy()), _bits(ref_out)), f"{label} {what}: forward"
        assert np.array_equal(_bits(gr.cpu().numpy()), _bits(ref_gr)), f"{label} {what}: grad_radial"
        check_grad_coupling(gc.cpu().numpy(), ref_gc, f"{label} {what}: grad_coupling")


def test_hip_graph_capture_and_replay(dev):
    """The whole step (asynchronous CSR build, forward, backward; also the
    normalised pair) captured in one HIP graph and replayed several times, with
    eager work and synchronisations between replays: every replay equals the
    eager result bitwise.  None of the calls allocates, synchronises or
    records a memset when given its buffers."""
    w = synthetic.custom("graph", 300, 20000, 32, seed=4242, envelope=True)
    x = synthetic.make_inputs(w)
    N, E, C = w.n_nodes, w.n_edges, w.channels
    say("[gpu] HIP graph capture of build + forward + backward")
    t = {k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "env",
                                                      "grad_out")}
    csr = zs.Csr(torch.empty(N + 1, dtype=torch.int32, device=dev),
                 torch.empty(E, dtype=torch.int32, device=dev),
                 torch.empty(E, dtype=torch.int32, device=dev), N,
                 torch.empty(N, dtype=torch.int32, device=dev))
    ws = torch.empty(zs.zs_csr_workspace_bytes(E, N), dtype=torch.uint8, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((N, 16, C), device=dev)
    gc = torch.empty((E, 15), device=dev)
    gr = torch.empty((E, 3, C), device=dev)

    def step():
        zs.zs_build_csr(t["dst"], N, workspace=ws, out=csr, bad_flag=flag)
        zs.zs_forward(t["coupling"], t["radial"], csr, out=out)
        zs.zs_backward(t["grad_out"], t["coupling"], t["radial"], csr, grad_coupling=gc,
                       grad_radial=gr)
        y, o, nrm = zs.zs_forward_normalized(t["coupling"], t["radial"], t["env"], csr)
        grads = zs.zs_backward_normalized(t["grad_out"], o, nrm, t["coupling"], t["radial"], csr)
        return [csr.rowptr, csr.perm, csr.dst32, csr.order, out, gc, gr, y, o, nrm, *grads]

    names = ("rowptr", "perm", "dst32", "order", "out", "gc", "gr", "y", "out_n", "norm", "gc_n",
             "gr_n", "genv", "gdeg")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        eager = [a.clone() for a in step()]   # warm-up on a side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    for rep in range(4):
        for a in captured:
            a.fill_(-7)   # eager work between replays, and a clobber the replay must undo
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, captured, eager):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {rep}: {name}"
        assert int(flag.item()) == 0
    ref_out = oracle.forward(x["coupling"], x["radial"], x["dst"], N)
    assert np.array_equal(_bits(out.cpu().numpy()), _bits(ref_out))


def test_node_order_is_a_schedule_only(dev):
    """The forward with the node schedule, without it (NULL), with a random
    permutation of the nodes, and with an order whose entries are partly not
    nodes: the first three are bitwise equal to the oracle; the last skips the
    positions that hold no node (range-checked, no access outside the
    buffers) and leaves those nodes' rows as they were."""
    N, E, C = 4096, 300000, 32
    w = synthetic.custom("order_sched", N, E, C, seed=6061, envelope=True)
    x = synthetic.make_inputs(w, with_grad=False)
    x["dst"] = heavy_destinations(E, N, seed=6061)
    say(f"[gpu] node order as a schedule: N={N} E={E} C={C}")
    dst = torch.from_numpy(x["dst"]).to(dev)
    cpl = torch.from_numpy(x["coupling"]).to(dev)
    rad = torch.from_numpy(x["radial"]).to(dev)
    csr = zs.zs_build_csr(dst, N)
    with_order = zs.zs_forward(cpl, rad, csr)
    without = zs.zs_forward(cpl, rad, csr._replace(order=None))
    shuffled = torch.from_numpy(np.random.default_rng(6062).permutation(N).astype(np.int32)).to(dev)
    any_perm = zs.zs_forward(cpl, rad, csr._replace(order=shuffled))
    bad = csr.order.clone()
    dropped = bad[:6].clone()                       # six of the highest-degree nodes
    bad[:3] = -1
    bad[3:6] = N + 3
    partial = zs.zs_forward(cpl, rad, csr._replace(order=bad),
                            out=torch.full((N, 16, C), float("nan"), device=dev))
    torch.cuda.synchronize()
    ref = oracle.forward(x["coupling"], x["radial"], x["dst"], N)
    assert np.array_equal(_bits(with_order.cpu().numpy()), _bits(ref))
    assert np.array_equal(_bits(without.cpu().numpy()), _bits(ref))
    assert np.array_equal(_bits(any_perm.cpu().numpy()), _bits(ref))
    got = partial.cpu().numpy()
    skip = np.zeros(N, dtype=bool)
    skip[dropped.cpu().numpy()] = True
    assert np.all(np.isnan(got[skip]))
    assert np.array_equal(_bits(got[~skip]), _bits(ref[~skip]))
