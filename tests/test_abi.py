"""The C ABI library: loads, exports what include/zs.h declares, and rejects bad
arguments on the host before any HIP call (CPU only: no compute is launched)."""
import ctypes
import subprocess

import pytest

import edge_node_scatter_amd as zs

ZS_ERR_NULL, ZS_ERR_SHAPE, ZS_ERR_INDEX = -1, -2, -3
ZS_ERR_UNSUPPORTED, ZS_ERR_ALIAS, ZS_ERR_WORKSPACE = -4, -5, -6
ZS_ERR_SCRATCH = -8

# Fake device addresses: every call below fails its host-side checks, so none
# of these is ever dereferenced or handed to HIP.
A = 0x7F0000000000
B = 0x7F1000000000
C_ = 0x7F2000000000
D = 0x7F3000000000
W = 0x7F4000000000
X = 0x7F5000000000


@pytest.fixture(scope="module")
def lib():
    return zs.load()


def test_header_symbols_exported(lib):
    declared = zs.declared_symbols()
    assert set(declared) == {"zs_status_string", "zs_csr_workspace_bytes", "zs_build_csr",
                             "zs_build_csr_noalloc", "zs_forward", "zs_backward", "zs_forward_strided",
                             "zs_backward_strided", "zs_forward_normalized",
                             "zs_backward_normalized"}
    out = subprocess.check_output(["nm", "-D", "--defined-only", zs.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for s in range(-8, 1):
        assert zs.status_string(s)
    assert zs.status_string(-99) == "unknown status"


def test_workspace_bytes(lib):
    assert zs.zs_csr_workspace_bytes(-1, 10) == 0
    assert zs.zs_csr_workspace_bytes(10, 0) == 0
    assert zs.zs_csr_workspace_bytes(647170, 4096) >= 4096 * 4
    assert zs.zs_csr_workspace_bytes(2600000, 16384) % 256 == 0


def test_build_csr_rejects(lib):
    def f(dst, e, n, rowptr, perm, dst32, ws, nbytes, flag=None, order=None):
        return lib.zs_build_csr(dst, e, n, rowptr, perm, dst32, order, ws, nbytes, flag, None)
    MB = 1 << 20
    assert f(A, 10, 0, B, C_, D, W, MB) == ZS_ERR_SHAPE
    assert f(A, -1, 4, B, C_, D, W, MB) == ZS_ERR_SHAPE
    assert f(None, 10, 4, B, C_, D, W, MB) == ZS_ERR_NULL
    assert f(A, 10, 4, None, C_, D, W, MB) == ZS_ERR_NULL
    assert f(A + 4, 10, 4, B, C_, D, W, MB) == ZS_ERR_UNSUPPORTED   # int64 misaligned
    assert f(A, 10, 4, B, C_, D, W, MB, X + 2) == ZS_ERR_UNSUPPORTED  # flag misaligned
    assert f(A, 10, 4, A + 8, C_, D, W, MB) == ZS_ERR_ALIAS         # rowptr inside dst
    assert f(A, 10, 4, B, B + 8, D, W, MB) == ZS_ERR_ALIAS          # perm over rowptr
    assert f(A, 10, 4, B, C_, D, W, MB, C_ + 4) == ZS_ERR_ALIAS     # flag inside perm
    assert f(A, 10, 4, B, C_, D, None, 0) == ZS_ERR_WORKSPACE
    assert f(A, 10, 4, B, C_, D, W, 16) == ZS_ERR_WORKSPACE
    assert f(A, 10, 4, B, C_, D, W + 4, MB) == ZS_ERR_UNSUPPORTED   # workspace alignment
    assert f(A, 10, 4, B, C_, D, A, MB) == ZS_ERR_ALIAS            # workspace over dst
    assert f(A, 10, 4, B, C_, D, W, MB, W + 64) == ZS_ERR_ALIAS     # flag inside workspace
    assert f(A, 10, 4, B, C_, D, W, MB, None, X + 2) == ZS_ERR_UNSUPPORTED   # order misaligned
    assert f(A, 10, 4, B, C_, D, W, MB, None, C_ + 8) == ZS_ERR_ALIAS    # order inside perm
    assert f(A, 10, 4, B, C_, D, W, MB, X, X) == ZS_ERR_ALIAS            # order over flag
    assert f(A, 10, 4, B, C_, D, W, MB, None, W + 256) == ZS_ERR_ALIAS   # order in workspace


def test_noalloc_limit_matches_the_header():
    import re
    m = re.search(r"#define ZS_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(zs.HEADER_PATH).read())
    assert m and int(m.group(1)) << int(m.group(2)) == zs.NOALLOC_SCRATCH_BYTES


def test_build_csr_noalloc_rejects(lib):
    """The same host checks as zs_build_csr, then the scratch limit: sizes whose
    workspace exceeds the fixed buffer are refused before any HIP call."""
    def f(dst, e, n, rowptr, perm, dst32, flag=None, order=None):
        return lib.zs_build_csr_noalloc(dst, e, n, rowptr, perm, dst32, order, flag, None)
    assert f(A, 10, 0, B, C_, D) == ZS_ERR_SHAPE
    assert f(None, 10, 4, B, C_, D) == ZS_ERR_NULL
    assert f(A + 4, 10, 4, B, C_, D) == ZS_ERR_UNSUPPORTED
    assert f(A, 10, 4, A + 8, C_, D) == ZS_ERR_ALIAS
    assert f(A, 10, 4, B, C_, D, C_ + 4) == ZS_ERR_ALIAS
    assert f(A, 10, 4, B, C_, D, None, D + 4) == ZS_ERR_ALIAS     # order inside dst32
    limit = zs.NOALLOC_SCRATCH_BYTES
    assert zs.zs_csr_workspace_bytes(2600000, 16384) <= limit     # the 16384-node frame fits
    big = 5_000_000
    assert zs.zs_csr_workspace_bytes(big, 4096) > limit
    assert f(A, big, 4096, B, C_, D) == ZS_ERR_SCRATCH
    assert "scratch" in zs.status_string(ZS_ERR_SCRATCH)


def test_forward_rejects(lib):
    f = lib.zs_forward
    assert f(A, B, C_, D, None, 4, 10, 0, X, None) == ZS_ERR_SHAPE
    assert f(A, B, C_, D, None, 4, 10, 1025, X, None) == ZS_ERR_SHAPE
    assert f(A, B, C_, D, None, 0, 10, 32, X, None) == ZS_ERR_SHAPE
    assert f(A, B, C_, D, None, 4, -2, 32, X, None) == ZS_ERR_SHAPE
    assert f(None, B, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_NULL
    assert f(A, B, C_, D, None, 4, 10, 32, None, None) == ZS_ERR_NULL
    assert f(A, B + 2, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_UNSUPPORTED
    assert f(A, B, C_, D, None, 4, 10, 32, B + 64, None) == ZS_ERR_ALIAS            # out over radial
    assert f(A, B, C_, D, None, 4, 10, 32, A, None) == ZS_ERR_ALIAS                 # out over coupling
    O = X + (1 << 20)
    assert f(A, B, C_, D, O + 2, 4, 10, 32, X, None) == ZS_ERR_UNSUPPORTED   # order misaligned
    assert f(A, B, C_, D, X + 8, 4, 10, 32, X, None) == ZS_ERR_ALIAS         # order inside out


def test_backward_rejects(lib):
    f = lib.zs_backward
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 10, 0, W, X, None) == ZS_ERR_SHAPE
    assert f(None, B, C_, D, D + 4096, D + 8192, 4, 10, 32, W, X, None) == ZS_ERR_NULL
    assert f(A, B, C_, None, D + 4096, D + 8192, 4, 10, 32, W, X, None) == ZS_ERR_NULL   # dst32
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 10, 32, W, None, None) == ZS_ERR_NULL
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 10, 32, W + 1, X, None) == ZS_ERR_UNSUPPORTED
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 10, 32, W, W + 16, None) == ZS_ERR_ALIAS
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 10, 32, A, X, None) == ZS_ERR_ALIAS
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 10, 32, W, C_ + 256, None) == ZS_ERR_ALIAS
    # no edges: nothing to write, returns before touching the device
    assert f(A, B, C_, D, D + 4096, D + 8192, 4, 0, 32, W, X, None) == 0


def test_strided_rejects(lib):
    f, b = lib.zs_forward_strided, lib.zs_backward_strided
    assert f(A, -1, B, 96, 32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE      # negative stride
    assert f(A, 15, B, -96, 32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE
    assert f(A, 15, B, 96, -32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE
    assert f(A, 46, B, 160, 32, C_, D, None, 4, 10, 0, X, None) == ZS_ERR_SHAPE      # channels
    # views whose extent overflows int64 or passes 2^60 floats
    big = 1 << 62
    assert f(A, big, B, 96, 32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE
    assert f(A, 15, B, big, 32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE
    assert f(A, 15, B, 96, big, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE
    assert f(A, (1 << 60) // 9 + 1, B, 96, 32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_SHAPE
    assert b(A, B, 46, C_, big, 32, D, D + 4096, D + 8192, 4, 10, 32, W, X, None) == ZS_ERR_SHAPE
    assert f(None, 46, B, 160, 32, C_, D, None, 4, 10, 32, X, None) == ZS_ERR_NULL
    # out inside the strided radial extent (9*160 + 2*32 + 32 floats) -> alias
    assert f(A, 46, B, 160, 32, C_, D, None, 4, 10, 32, B + 4 * 1500, None) == ZS_ERR_ALIAS
    # out inside the strided coupling extent (9*46 + 15 floats) -> alias
    assert f(A, 46, B, 160, 32, C_, D, None, 4, 10, 32, A + 4 * 420, None) == ZS_ERR_ALIAS
    assert b(A, B, -46, C_, 160, 32, D, D + 4096, D + 8192, 4, 10, 32, W, X, None) == ZS_ERR_SHAPE
    assert b(A, B, 46, C_, 160, 32, D, D + 4096, D + 8192, 4, 10, 32, W, C_ + 4 * 1500,
             None) == ZS_ERR_ALIAS
    assert b(A, B, 46, C_, 160, 32, D, D + 4096, D + 8192, 4, 0, 32, W, X, None) == 0


def test_normalized_rejects(lib):
    # zs_forward_normalized(coupling, radial, env, rowptr, perm, order, N, E, C, y, out, norm,
    #                       stream)
    f = lib.zs_forward_normalized
    Y, O, NR = X, X + (1 << 20), X + (2 << 20)
    assert f(A, B, W, C_, D, None, 4, 10, 0, Y, O, NR, None) == ZS_ERR_SHAPE
    assert f(A, B, None, C_, D, None, 4, 10, 32, Y, O, NR, None) == ZS_ERR_NULL      # env
    assert f(A, B, W, C_, D, None, 4, 10, 32, Y, O, None, None) == ZS_ERR_NULL      # norm
    assert f(A, B, W, C_, D, None, 4, 10, 32, None, O, NR, None) == ZS_ERR_NULL     # y
    assert f(A, B, W + 2, C_, D, None, 4, 10, 32, Y, O, NR, None) == ZS_ERR_UNSUPPORTED
    assert f(A, B, W, C_, D, None, 4, 10, 32, Y, O + 1, NR, None) == ZS_ERR_UNSUPPORTED
    assert f(A, B, W, C_, D, None, 4, 10, 32, Y, Y + 64, NR, None) == ZS_ERR_ALIAS  # out over y
    assert f(A, B, W, C_, D, None, 4, 10, 32, Y, O, O + 8, None) == ZS_ERR_ALIAS    # norm over out
    assert f(A, B, W, C_, D, None, 4, 10, 32, Y, None, Y + 4, None) == ZS_ERR_ALIAS  # norm over y
    assert f(A, B, W, C_, D, None, 4, 10, 32, Y, O, W + 4, None) == ZS_ERR_ALIAS    # norm over env
    assert f(A, B, W, C_, D, None, 4, 10, 32, B + 64, O, NR, None) == ZS_ERR_ALIAS  # y over radial
    assert f(A, B, W, C_, D, Y + 16, 4, 10, 32, Y, O, NR, None) == ZS_ERR_ALIAS    # order in y
    assert f(A, B, W, C_, D, X + (5 << 20) + 1, 4, 10, 32, Y, O, NR, None) == ZS_ERR_UNSUPPORTED
    # zs_backward_normalized(gy, out, norm, coupling, radial, dst32, rowptr, perm, N, E, C,
    #                        gc, gr, genv, gdeg, stream)
    b = lib.zs_backward_normalized
    GY, OU, NM = A, A + (1 << 20), A + (2 << 20)
    GC, GR, GE, GD = X, X + (1 << 20), X + (2 << 20), X + (3 << 20)
    args = [GY, OU, NM, B, C_, D, D + 4096, D + 8192, 4, 10, 32, GC, GR, GE, GD, None]

    def call(**kw):
        a = list(args)
        names = ["gy", "out", "norm", "cpl", "rad", "dst32", "rowptr", "perm", "N", "E", "C",
                 "gc", "gr", "ge", "gd", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return b(*a)
    assert call(C=0) == ZS_ERR_SHAPE
    assert call(E=-1) == ZS_ERR_SHAPE
    assert call(gd=None) == ZS_ERR_NULL
    assert call(out=None) == ZS_ERR_NULL
    assert call(ge=None) == ZS_ERR_NULL
    assert call(gd=GD + 2) == ZS_ERR_UNSUPPORTED
    assert call(ge=GE + 1) == ZS_ERR_UNSUPPORTED
    assert call(ge=GC + 8) == ZS_ERR_ALIAS          # grad_env inside grad_coupling
    assert call(gd=OU + 16) == ZS_ERR_ALIAS         # grad_deg over out
    assert call(gr=GY) == ZS_ERR_ALIAS              # grad_radial over grad_y
    assert call(gc=NM) == ZS_ERR_ALIAS              # grad_coupling over norm


def test_band_view_helper():
    import torch
    band = torch.arange(5 * 46, dtype=torch.float32).reshape(5, 46)
    c = zs.coupling_from_band(band)
    assert c.shape == (5, 15) and c.stride() == (46, 1)
    assert torch.equal(c[:, 0], band[:, 16]) and torch.equal(c[:, 14], band[:, 30])


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        zs.zs_build_csr(torch.zeros(3, dtype=torch.int64), 4)


def test_c_client_links_against_the_header(c_client, tmp_path):
    """The header compiles as C11 with -Wall -Werror, and a plain C program
    links against libzs.so alone for every call it makes."""
    out = subprocess.check_output(["nm", "-u", c_client], text=True)
    undefined = {line.split()[-1] for line in out.splitlines()}
    for name in ("zs_status_string", "zs_csr_workspace_bytes", "zs_build_csr", "zs_forward",
                 "zs_backward"):
        assert name in undefined, name
    # argument and file errors are handled before any HIP call
    r = subprocess.run([c_client], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    r = subprocess.run([c_client, str(tmp_path / "missing.bin"), str(tmp_path / "o.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1
    short = tmp_path / "short.bin"
    short.write_bytes(b"\x01\x00")
    r = subprocess.run([c_client, str(short), str(tmp_path / "o.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "short header" in r.stderr


def test_binding_rejects_wrong_buffers():
    """Caller-supplied outputs, workspace and CSR arrays must be dense arrays
    of exactly the shape the kernels address (checked before any call)."""
    import torch
    cpu = torch.device("cpu")
    ok = torch.empty((4, 16, 8))
    assert zs._buffer(ok, "out", (4, 16, 8), torch.float32, cpu) is ok
    with pytest.raises(ValueError, match="shape"):
        zs._buffer(torch.empty((3, 16, 8)), "out", (4, 16, 8), torch.float32, cpu)
    with pytest.raises(TypeError):
        zs._buffer(torch.empty((4, 16, 8), dtype=torch.float64), "out", (4, 16, 8),
                   torch.float32, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        zs._buffer(torch.empty((4, 8, 16)).transpose(1, 2), "out", (4, 16, 8), torch.float32, cpu)
    with pytest.raises(ValueError, match="tensor on"):
        zs._buffer(ok, "out", (4, 16, 8), torch.float32, torch.device("cuda", 0))
    csr = zs.Csr(torch.empty(5, dtype=torch.int32), torch.empty(7, dtype=torch.int32),
                 torch.empty(7, dtype=torch.int32), 4)
    zs._csr_buffers(csr, 7, cpu)
    with pytest.raises(ValueError, match="csr.perm"):
        zs._csr_buffers(csr, 8, cpu)
    with pytest.raises(ValueError, match="csr.rowptr"):
        zs._csr_buffers(csr._replace(n_nodes=5), 7, cpu)
