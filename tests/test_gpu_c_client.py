"""The C ABI used from plain C (tests/c_abi_client.c: HIP runtime + libzs, no
Python or torch in the process): the stable CSR build, forward and backward on
the default stream, compared with the oracle to the same bar as the Python
binding's parity tests (bitwise CSR, forward and grad_radial; grad_coupling
within 1e-6 + 1e-5 |ref|)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu
ATOL, RTOL = 1e-6, 1e-5

CASES = [
    # label, N, E, C
    ("tiny", 64, 2000, 32),
    ("sparse_c20", 3000, 7001, 20),   # many empty nodes, channels not a multiple of 4
    ("no_edges", 5, 0, 8),
]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _write_input(path, x, N, E, C):
    with open(path, "wb") as f:
        np.array([N, E, C], dtype="<i8").tofile(f)
        for k in ("dst", "coupling", "radial", "grad_out"):
            np.ascontiguousarray(x[k]).tofile(f)


def _read_output(path, N, E, C):
    raw = open(path, "rb").read()
    sizes = [("rowptr", np.int32, N + 1), ("perm", np.int32, E), ("out", np.float32, N * 16 * C),
             ("gc", np.float32, E * 15), ("gr", np.float32, E * 3 * C)]
    res, off = {}, 0
    for name, dt, n in sizes:
        res[name] = np.frombuffer(raw, dtype=dt, count=n, offset=off)
        off += n * np.dtype(dt).itemsize
    assert off == len(raw), f"output file holds {len(raw)} bytes, expected {off}"
    return res


@pytest.mark.parametrize("label,N,E,C", CASES, ids=[c[0] for c in CASES])
def test_c_client_matches_oracle(c_client, tmp_path, label, N, E, C):
    print(f"c client: {label} N={N} E={E} C={C}", flush=True)
    sys.stdout.flush()
    x = synthetic.make_inputs(synthetic.custom(label, N, E, C, seed=6000 + N + E + C))
    inp, outp = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_input(inp, x, N, E, C)
    r = subprocess.run([c_client, inp, outp], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client exit {r.returncode}: {r.stderr}"
    res = _read_output(outp, N, E, C)

    rowptr, perm = oracle.csr(x["dst"], N)
    assert np.array_equal(res["rowptr"], rowptr)
    assert np.array_equal(res["perm"], perm)
    out = oracle.forward(x["coupling"], x["radial"], x["dst"], N).reshape(-1)
    assert np.array_equal(_bits(res["out"]), _bits(out))
    if E == 0:
        return
    gc, gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    assert np.array_equal(_bits(res["gr"]), _bits(gr.reshape(-1)))
    ref = gc.reshape(-1).astype(np.float64)
    diff = np.abs(res["gc"].astype(np.float64) - ref)
    assert np.all(diff <= ATOL + RTOL * np.abs(ref))


def test_c_client_reports_bad_destination(c_client, tmp_path):
    """A destination outside [0, N) comes back as the ABI's index error, with
    its status text, and the client exits non-zero without writing results."""
    N, E, C = 16, 100, 4
    x = synthetic.make_inputs(synthetic.custom("bad_dst", N, E, C, seed=6100))
    x["dst"] = x["dst"].copy()
    x["dst"][37] = N
    inp, outp = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_input(inp, x, N, E, C)
    r = subprocess.run([c_client, inp, outp], capture_output=True, text=True, timeout=120)
    assert r.returncode == 3, r.stderr
    assert "zs_build_csr" in r.stderr and "(-3)" in r.stderr
    assert not os.path.exists(outp)
