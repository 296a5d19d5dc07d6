"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something the pages or the mathematics fix:

* brute force: the message surface materialised explicitly and summed by a
  dense incidence-matrix product (a library matmul), in fp64;
* the same composition evaluated with numpy fp32 ops in edge order, which the
  pages say is the addition order of the reference (index_add);
* closed forms: all-ones inputs count degrees; C = 1 with unit coupling is a
  plain segment sum; one edge gives an outer product; the worked layout
  example from the review of the backward's padded channel loads;
* invariants: scalar row 0 is +0, scaling by powers of two commutes exactly,
  additivity and edge-permutation invariance on exactly representable inputs,
  conservation of the total message;
* the backward: adjoint identity, an explicit Jacobian on a tiny problem,
  finite differences, exact rational sums for the channel reduction, the
  fp32 grad_radial order, and insensitivity to upstream row 0;
* the CSR: a library stable argsort and a brute-force scan;
* the degree normalisation: unit envelopes (neighbour counts, closed-form
  1/sqrt), exact halving when every envelope is multiplied by 4, the fp64
  evaluation, finite differences of all three gradients, and insensitivity
  to upstream rows that cannot matter.

Sizes are small so the whole set runs in a few seconds; ``test_oracle_pins``
runs it on the committed oracle and ``test_oracle_mutants`` runs it on copies
of the oracle with planted mistakes, each of which must fail at least one pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle as _oracle_mod

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 2.0 ** -24          # unit roundoff of fp32
DEG = np.array([math.isqrt(r) for r in range(16)])   # degree l of padded row r


def _rng(seed):
    return np.random.default_rng(seed)


def _problem(seed, E, N, C, dst=None, dyadic=False):
    g = _rng(seed)
    if dst is None:
        dst = g.integers(0, N, size=E).astype(np.int64)
    if dyadic:
        cpl = (g.integers(-64, 65, size=(E, 15)) / 64.0).astype(np.float32)
        rad = (g.integers(-64, 65, size=(E, 3, C)) / 64.0).astype(np.float32)
        gout = (g.integers(-64, 65, size=(N, 16, C)) / 64.0).astype(np.float32)
    else:
        cpl = g.uniform(-1, 1, size=(E, 15)).astype(np.float32)
        rad = g.standard_normal(size=(E, 3, C)).astype(np.float32)
        gout = g.standard_normal(size=(N, 16, C)).astype(np.float32)
    return dst, cpl, rad, gout


def _message64(cpl, rad):
    """Explicit (E,15,C) message in fp64; row r uses radial slot isqrt(r)-1."""
    return cpl.astype(np.float64)[:, :, None] * rad.astype(np.float64)[:, DEG[1:] - 1, :]


def _incidence(dst, N):
    A = np.zeros((N, len(dst)))
    A[dst, np.arange(len(dst))] = 1.0
    return A


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype == np.float32 else np.uint64)


def _assert_bitwise(a, b, what):
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    bad = np.count_nonzero(_bits(a) != _bits(b))
    assert bad == 0, f"{what}: {bad} elements differ bitwise"


def _round_f32(x: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 of an exact rational."""
    f = np.float32(float(x))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - x)
        key = (d, int(_bits(np.array([cand]))[0]) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


# --------------------------------------------------------------------------- forward
def pin_forward_bruteforce(orc):
    for seed, (E, N, C) in enumerate([(257, 13, 7), (400, 3, 5), (64, 40, 9)]):
        dst, cpl, rad, _ = _problem(100 + seed, E, N, C)
        M = _message64(cpl, rad)
        A = _incidence(dst, N)
        ref = (A @ M.reshape(E, -1)).reshape(N, 15, C)
        mag = (A @ np.abs(M).reshape(E, -1)).reshape(N, 15, C)
        deg = np.bincount(dst, minlength=N)[:, None, None]
        o64 = orc.forward(cpl, rad, dst, N, dtype=np.float64)
        assert np.all(o64[:, 0] == 0.0), "fp64 row 0 not zero"
        assert np.all(np.abs(o64[:, 1:] - ref) <= 1e-13 * (mag + 1e-300)), "fp64 forward vs brute force"
        o32 = orc.forward(cpl, rad, dst, N).astype(np.float64)
        assert np.all(o32[:, 0] == 0.0), "fp32 row 0 not zero"
        bound = (deg + 2) * U32 * mag + 1e-30
        assert np.all(np.abs(o32[:, 1:] - ref) <= bound), "fp32 forward outside the rounding bound"


def pin_forward_fp32_edge_order(orc):
    """numpy fp32: multiply, then add in increasing edge order (index_add order)."""
    E, N, C = 300, 11, 6
    dst, cpl, rad, _ = _problem(7, E, N, C)
    ref = np.zeros((N, 16, C), dtype=np.float32)
    for e in range(E):
        msg = cpl[e][:, None] * rad[e][DEG[1:] - 1]          # fp32 products
        ref[dst[e], 1:] = ref[dst[e], 1:] + msg                # fp32 adds
    _assert_bitwise(orc.forward(cpl, rad, dst, N), ref, "forward vs fp32 edge-order composition")


def pin_forward_degree_count(orc):
    E, N, C = 500, 37, 3
    dst = _rng(3).integers(0, N - 5, size=E).astype(np.int64)      # last 5 nodes empty
    out = orc.forward(np.ones((E, 15), np.float32), np.ones((E, 3, C), np.float32), dst, N)
    deg = np.bincount(dst, minlength=N).astype(np.float32)
    assert np.array_equal(out[:, 1:], np.broadcast_to(deg[:, None, None], (N, 15, C))), "degree count"
    assert np.all(_bits(out[:, 0]) == 0), "row 0 must be +0"


def pin_forward_segment_sum(orc):
    """C = 1 and unit coupling: each row is a segment sum of one radial slot."""
    E, N = 200, 9
    dst, _, rad, _ = _problem(11, E, N, 1)
    out = orc.forward(np.ones((E, 15), np.float32), rad, dst, N)
    for r in range(1, 16):
        ref = np.zeros(N, dtype=np.float32)
        np.add.at(ref, dst, rad[:, DEG[r] - 1, 0])            # unbuffered, in index order
        _assert_bitwise(out[:, r, 0], ref, f"segment sum row {r}")


def pin_forward_single_edge(orc):
    dst, cpl, rad, _ = _problem(5, 1, 4, 8, dst=np.array([2]))
    out = orc.forward(cpl, rad, dst, 4)
    ref = np.zeros((4, 16, 8), dtype=np.float32)
    for r in range(1, 16):
        ref[2, r] = cpl[0, r - 1] * rad[0, DEG[r] - 1]
    _assert_bitwise(out, ref, "single edge outer product")


def pin_forward_signed_zero(orc):
    """Accumulators start at +0: a -0 message, empty nodes and row 0 give +0."""
    E, N, C = 6, 3, 4
    dst = np.array([0, 0, 1, 1, 1, 0], dtype=np.int64)
    cpl = np.full((E, 15), -0.0, dtype=np.float32)
    rad = np.ones((E, 3, C), dtype=np.float32)
    out = orc.forward(cpl, rad, dst, N)
    assert np.all(_bits(out) == 0), "-0 messages must accumulate to +0"


def pin_forward_pow2_scaling(orc):
    E, N, C = 300, 7, 5
    dst, cpl, rad, _ = _problem(13, E, N, C)
    base = orc.forward(cpl, rad, dst, N)
    _assert_bitwise(orc.forward(cpl * np.float32(2), rad, dst, N), base * np.float32(2), "F(2x)=2F(x)")
    _assert_bitwise(orc.forward(cpl, rad * np.float32(0.25), dst, N), base * np.float32(0.25),
                    "F(y/4)=F(y)/4")


def pin_forward_additivity_and_permutation(orc):
    """Dyadic inputs keep every product and partial sum exact in fp32."""
    E, N, C = 250, 6, 4
    dst, c1, rad, _ = _problem(17, E, N, C, dyadic=True)
    _, c2, _, _ = _problem(18, E, N, C, dyadic=True)
    f1, f2 = orc.forward(c1, rad, dst, N), orc.forward(c2, rad, dst, N)
    _assert_bitwise(orc.forward(c1 + c2, rad, dst, N), f1 + f2, "additivity")
    p = _rng(19).permutation(E)
    _assert_bitwise(orc.forward(c1[p], rad[p], dst[p], N), f1, "edge permutation invariance")


def pin_forward_total(orc):
    E, N, C = 800, 20, 6
    dst, cpl, rad, _ = _problem(23, E, N, C)
    tot = orc.forward(cpl, rad, dst, N, dtype=np.float64)[:, 1:].sum(axis=0)
    M = _message64(cpl, rad)
    ref = M.sum(axis=0)
    assert np.allclose(tot, ref, rtol=1e-12, atol=1e-12 * np.abs(M).sum(axis=0).max()), "total message"


def pin_forward_nodes_sample(orc):
    E, N, C = 400, 15, 5
    dst, cpl, rad, _ = _problem(29, E, N, C)
    full = orc.forward(cpl, rad, dst, N)
    nodes = np.array([0, 14, 3, 3, 7])
    _assert_bitwise(orc.forward_nodes(cpl, rad, dst, N, nodes), full[nodes], "sampled forward rows")


def pin_pages_layout_example(orc):
    """The review of the backward's padded channel loads works through a
    (777, 3, 40) radial tensor: 93,240 floats, the last edge's third slot
    starting at float 93,200.  Encode each radial float's flat index as its
    value and read it back through a one-hot coupling on a degree-3 row."""
    fx = _golden("layout_worked_example.txt")
    E, N, C = int(fx["edges"]), int(fx["nodes"]), int(fx["channels"])
    assert E * 3 * C == int(fx["radial_floats"])
    rad = np.arange(E * 3 * C, dtype=np.float32).reshape(E, 3, C)
    dst = _rng(31).integers(0, N, size=E).astype(np.int64)
    cpl = np.zeros((E, 15), dtype=np.float32)
    e_last = E - 1
    cpl[e_last, 9] = 1.0                          # row 10 has degree 3 -> slot 2
    out = orc.forward(cpl, rad, dst, N)
    start = int(fx["last_edge_slot2_start"])
    assert np.array_equal(out[dst[e_last], 10], np.arange(start, start + C, dtype=np.float32)), \
        "radial flat offset ((e*3)+slot)*C + c"
    # and the full composition at that shape against brute force
    _, cpl2, rad2, _ = _problem(37, E, N, C)
    ref = (_incidence(dst, N) @ _message64(cpl2, rad2).reshape(E, -1)).reshape(N, 15, C)
    got = orc.forward(cpl2, rad2, dst, N, dtype=np.float64)[:, 1:]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), "777x33x40 forward"


# --------------------------------------------------------------------------- backward
def pin_backward_adjoint(orc):
    E, N, C = 600, 17, 8
    dst, cpl, rad, g = _problem(41, E, N, C)
    F = orc.forward(cpl, rad, dst, N, dtype=np.float64)
    gc, gr = orc.backward(g, cpl, rad, dst, dtype=np.float64)
    lhs = float(np.sum(g.astype(np.float64) * F))
    scale = float(np.sum(np.abs(g[:, 1:].astype(np.float64)) *
                         (_incidence(dst, N) @ np.abs(_message64(cpl, rad)).reshape(E, -1)).reshape(N, 15, C)))
    x = float(np.sum(gc * cpl.astype(np.float64)))
    y = float(np.sum(gr * rad.astype(np.float64)))
    assert abs(lhs - x) <= 1e-12 * scale, "<g,F> vs <grad_coupling, coupling>"
    assert abs(lhs - y) <= 1e-12 * scale, "<g,F> vs <grad_radial, radial>"
    gc32, gr32 = orc.backward(g, cpl, rad, dst)
    assert abs(float(np.sum(gc32.astype(np.float64) * cpl)) - lhs) <= 1e-6 * scale
    assert abs(float(np.sum(gr32.astype(np.float64) * rad)) - lhs) <= 1e-6 * scale


def pin_backward_jacobian(orc):
    """Explicit Jacobian of the (linear-in-each-operand) forward on a tiny case."""
    E, N, C = 4, 3, 3
    dst, cpl, rad, g = _problem(43, E, N, C, dst=np.array([2, 0, 2, 1]))
    g64 = g.astype(np.float64).ravel()
    jx = np.zeros((E * 15, N * 16 * C))
    for i in range(E * 15):
        u = np.zeros(E * 15, dtype=np.float32)
        u[i] = 1.0
        jx[i] = orc.forward(u.reshape(E, 15), rad, dst, N, dtype=np.float64).ravel()
    jy = np.zeros((E * 3 * C, N * 16 * C))
    for i in range(E * 3 * C):
        u = np.zeros(E * 3 * C, dtype=np.float32)
        u[i] = 1.0
        jy[i] = orc.forward(cpl, u.reshape(E, 3, C), dst, N, dtype=np.float64).ravel()
    gc, gr = orc.backward(g, cpl, rad, dst, dtype=np.float64)
    assert np.allclose(gc.ravel(), jx @ g64, rtol=1e-13, atol=1e-13), "grad_coupling vs J^T g"
    assert np.allclose(gr.ravel(), jy @ g64, rtol=1e-13, atol=1e-13), "grad_radial vs J^T g"
    gc32, gr32 = orc.backward(g, cpl, rad, dst)
    assert np.allclose(gc32.ravel(), jx @ g64, rtol=4 * U32, atol=1e-30), "fp32 grad_coupling"
    assert np.allclose(gr32.ravel(), jy @ g64, rtol=1e-5, atol=1e-6), "fp32 grad_radial"


def pin_backward_finite_difference(orc):
    E, N, C = 900, 12, 6
    dst, cpl, rad, g = _problem(47, E, N, C)
    gc, gr = orc.backward(g, cpl, rad, dst, dtype=np.float64)
    g64 = g.astype(np.float64)

    def loss(c, r):
        return float(np.sum(g64 * orc.forward(c, r, dst, N, dtype=np.float64)))

    rng = _rng(48)
    h = np.float32(0.5)
    for _ in range(12):
        e, j = rng.integers(E), rng.integers(15)
        cp, cm = cpl.copy(), cpl.copy()
        cp[e, j] += h
        cm[e, j] -= h
        fd = (loss(cp, rad) - loss(cm, rad)) / (float(cp[e, j]) - float(cm[e, j]))
        assert abs(fd - gc[e, j]) <= 1e-9 * (1 + abs(gc[e, j])), "FD grad_coupling"
        s, c = rng.integers(3), rng.integers(C)
        rp, rm = rad.copy(), rad.copy()
        rp[e, s, c] += h
        rm[e, s, c] -= h
        fd = (loss(cpl, rp) - loss(cpl, rm)) / (float(rp[e, s, c]) - float(rm[e, s, c]))
        assert abs(fd - gr[e, s, c]) <= 1e-9 * (1 + abs(gr[e, s, c])), "FD grad_radial"


def pin_grad_coupling_correctly_rounded(orc):
    """The channel sum, taken exactly (rationals) and rounded once to fp32."""
    E, N, C = 40, 5, 33
    dst, cpl, rad, g = _problem(53, E, N, C)
    gc, _ = orc.backward(g, cpl, rad, dst)
    for e in range(E):
        for r in range(1, 16):
            exact = sum(Fraction(float(g[dst[e], r, c])) * Fraction(float(rad[e, DEG[r] - 1, c]))
                        for c in range(C))
            want = _round_f32(exact)
            assert _bits(np.array([gc[e, r - 1]]))[0] == _bits(np.array([want]))[0], \
                f"grad_coupling[{e},{r - 1}] not the rounded exact sum"


def pin_grad_radial_fp32_order(orc):
    """grad_radial adds each degree's rows in increasing r, fp32 mul then add."""
    E, N, C = 120, 7, 5
    dst, cpl, rad, g = _problem(59, E, N, C)
    _, gr = orc.backward(g, cpl, rad, dst)
    ref = np.zeros((E, 3, C), dtype=np.float32)
    for e in range(E):
        for l in (1, 2, 3):
            acc = np.zeros(C, dtype=np.float32)
            for r in range(l * l, (l + 1) * (l + 1)):
                acc = acc + g[dst[e], r] * cpl[e, r - 1]
            ref[e, l - 1] = acc
    _assert_bitwise(gr, ref, "grad_radial order")
    gr64 = orc.backward(g, cpl, rad, dst, dtype=np.float64)[1]
    mag = np.zeros((E, 3, C))
    for l in (1, 2, 3):
        rows = list(range(l * l, (l + 1) * (l + 1)))
        mag[:, l - 1] = np.sum(np.abs(g[dst][:, rows].astype(np.float64) *
                                      cpl[:, [r - 1 for r in rows], None]), axis=1)
    assert np.all(np.abs(gr.astype(np.float64) - gr64) <= 9 * U32 * mag + 1e-30), "grad_radial bound"


def pin_grad_row0_ignored(orc):
    E, N, C = 90, 6, 4
    dst, cpl, rad, g = _problem(61, E, N, C)
    a = orc.backward(g, cpl, rad, dst)
    g2 = g.copy()
    g2[:, 0] = np.float32(1e30)
    b = orc.backward(g2, cpl, rad, dst)
    _assert_bitwise(a[0], b[0], "grad_coupling vs upstream row 0")
    _assert_bitwise(a[1], b[1], "grad_radial vs upstream row 0")


def pin_backward_edges_sample(orc):
    E, N, C = 150, 8, 5
    dst, cpl, rad, g = _problem(67, E, N, C)
    gc, gr = orc.backward(g, cpl, rad, dst)
    idx = np.array([0, 149, 77, 77])
    sc, sr = orc.backward_edges(g, cpl, rad, dst, idx)
    _assert_bitwise(sc, gc[idx], "sampled grad_coupling")
    _assert_bitwise(sr, gr[idx], "sampled grad_radial")


# --------------------------------------------------------------------------- CSR and errors
def pin_csr(orc):
    for seed, (E, N) in enumerate([(1000, 37), (0, 5), (50, 1), (300, 600)]):
        dst = _rng(71 + seed).integers(0, N, size=E).astype(np.int64)
        rowptr, perm = orc.csr(dst, N)
        assert np.array_equal(perm, np.argsort(dst, kind="stable").astype(np.int32)), "stable argsort"
        ref = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=N))]).astype(np.int32)
        assert np.array_equal(rowptr, ref), "rowptr"
    dst = _rng(79).integers(0, 6, size=40).astype(np.int64)
    rowptr, perm = orc.csr(dst, 6)
    brute = [e for n in range(6) for e in range(40) if dst[e] == n]
    assert list(perm) == brute, "brute-force CSR"


def pin_bad_index(orc):
    E, N, C = 10, 4, 3
    _, cpl, rad, g = _problem(83, E, N, C)
    for bad in (N, -1, 2 ** 40):
        dst = np.zeros(E, dtype=np.int64)
        dst[E // 2] = bad
        for call in (lambda: orc.forward(cpl, rad, dst, N),
                     lambda: orc.backward(g, cpl, rad, dst),
                     lambda: orc.csr(dst, N)):
            try:
                call()
            except _oracle_mod.OracleIndexError:
                continue
            raise AssertionError(f"destination {bad} accepted")


def _golden(name):
    fx = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                fx[k.strip()] = v.strip()
    return fx




# --------------------------------------------------------------------------- degree normalisation
def _norm_problem(seed, E, N, C):
    dst, cpl, rad, g = _problem(seed, E, N, C)
    env = _rng(seed + 1).uniform(0.05, 1.0, size=E).astype(np.float32)
    return dst, cpl, rad, g, env


def pin_norm_unit_envelope(orc):
    """Unit envelopes: deg = neighbour count, norm = 1/sqrt(count) (one fp32
    sqrt and one fp32 division), empty nodes get 0; y against fp64 brute force."""
    E, N, C = 400, 23, 6
    dst = _rng(91).integers(0, N - 3, size=E).astype(np.int64)        # 3 empty nodes
    _, cpl, rad, _ = _problem(92, E, N, C, dst=dst)
    y, out, norm = orc.forward_norm(cpl, rad, np.ones(E, np.float32), dst, N)
    cnt = np.bincount(dst, minlength=N).astype(np.float32)
    want = np.zeros(N, np.float32)
    nz = cnt > 0
    want[nz] = np.float32(1.0) / np.sqrt(cnt[nz])
    _assert_bitwise(norm, want, "norm with unit envelopes")
    ref = (_incidence(dst, N) @ _message64(cpl, rad).reshape(E, -1)).reshape(N, 15, C)
    ref = ref / np.where(cnt > 0, np.sqrt(cnt.astype(np.float64)), np.inf)[:, None, None]
    mag = (_incidence(dst, N) @ np.abs(_message64(cpl, rad)).reshape(E, -1)).reshape(N, 15, C)
    bound = (cnt[:, None, None] + 6) * U32 * mag / np.maximum(np.sqrt(cnt), 1)[:, None, None]
    assert np.all(np.abs(y[:, 1:].astype(np.float64) - ref) <= bound + 1e-30), "y vs brute force"
    assert np.all(_bits(y[:, 0]) == 0) and np.all(_bits(y[~nz]) == 0), "row 0 / empty nodes"


def pin_norm_envelope_scaling(orc):
    """Envelopes times 4: every degree times 4, norm halved exactly, y halved."""
    E, N, C = 300, 11, 5
    dst, cpl, rad, _, env = _norm_problem(93, E, N, C)
    y1, _, n1 = orc.forward_norm(cpl, rad, env, dst, N)
    y4, _, n4 = orc.forward_norm(cpl, rad, env * np.float32(4), dst, N)
    _assert_bitwise(n4, n1 * np.float32(0.5), "norm(4 env) = norm(env)/2")
    _assert_bitwise(y4, y1 * np.float32(0.5), "y(4 env) = y(env)/2")


def pin_norm_matches_fp64(orc):
    E, N, C = 500, 17, 7
    dst, cpl, rad, _, env = _norm_problem(94, E, N, C)
    y, _, norm = orc.forward_norm(cpl, rad, env, dst, N)
    y64, norm64 = orc.forward_norm(cpl, rad, env, dst, N, dtype=np.float64)
    assert np.allclose(norm, norm64, rtol=8 * U32, atol=0), "norm vs fp64"
    deg = np.bincount(dst, minlength=N)[:, None, None]
    absm = (_incidence(dst, N) @ np.abs(_message64(cpl, rad)).reshape(E, -1)).reshape(N, 15, C)
    bound = (deg + 6) * U32 * absm * norm64[:, None, None] + 1e-30
    assert np.all(np.abs(y[:, 1:] - y64[:, 1:]) <= bound), "y vs fp64"


def pin_norm_backward_finite_difference(orc):
    """Gradients of L = <gy, y> by central differences of the fp64 forward."""
    E, N, C = 240, 9, 4
    dst, cpl, rad, gy, env = _norm_problem(95, E, N, C)
    y, out, norm = orc.forward_norm(cpl, rad, env, dst, N)
    gc, gr, ge = orc.backward_norm(gy, out, norm, cpl, rad, dst)
    g64 = gy.astype(np.float64)

    def loss(c, r, v):
        return float(np.sum(g64 * orc.forward_norm(c, r, v, dst, N, dtype=np.float64)[0]))

    rng = _rng(96)
    for _ in range(10):
        e = rng.integers(E)
        h = np.float32(1.0 / 64)
        vp, vm = env.copy(), env.copy()
        vp[e] += h
        vm[e] -= h
        fd = (loss(cpl, rad, vp) - loss(cpl, rad, vm)) / (float(vp[e]) - float(vm[e]))
        assert abs(fd - ge[e]) <= 1e-4 * abs(fd) + 1e-5, f"grad_env[{e}]: {ge[e]} vs FD {fd}"
        j = rng.integers(15)
        cp, cm = cpl.copy(), cpl.copy()
        cp[e, j] += np.float32(0.5)
        cm[e, j] -= np.float32(0.5)
        fd = (loss(cp, rad, env) - loss(cm, rad, env)) / (float(cp[e, j]) - float(cm[e, j]))
        assert abs(fd - gc[e, j]) <= 1e-5 * abs(fd) + 1e-6, "grad_coupling (normalised)"
        s, c = rng.integers(3), rng.integers(C)
        rp, rm = rad.copy(), rad.copy()
        rp[e, s, c] += np.float32(0.5)
        rm[e, s, c] -= np.float32(0.5)
        fd = (loss(cpl, rp, env) - loss(cpl, rm, env)) / (float(rp[e, s, c]) - float(rm[e, s, c]))
        assert abs(fd - gr[e, s, c]) <= 1e-5 * abs(fd) + 1e-6, "grad_radial (normalised)"


def pin_norm_backward_zero_degree_rows(orc):
    """Upstream gradient on nodes without edges and on row 0 changes nothing."""
    E, N, C = 150, 12, 5
    dst = _rng(97).integers(0, N - 4, size=E).astype(np.int64)
    _, cpl, rad, gy = _problem(98, E, N, C, dst=dst)
    env = _rng(99).uniform(0.1, 1.0, size=E).astype(np.float32)
    y, out, norm = orc.forward_norm(cpl, rad, env, dst, N)
    a = orc.backward_norm(gy, out, norm, cpl, rad, dst)
    g2 = gy.copy()
    g2[N - 4:] = np.float32(7.0)
    g2[:, 0] = np.float32(-3.0)
    b = orc.backward_norm(g2, out, norm, cpl, rad, dst)
    for u, v, what in zip(a, b, ("grad_coupling", "grad_radial", "grad_env")):
        _assert_bitwise(u, v, what)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
