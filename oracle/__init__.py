"""CPU oracle for the GIE zonal scatter -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``zs_oracle.c`` (plain sequential C, built by
``gcc -O2 -ffp-contract=off``) through ctypes and shares no code with the HIP
library in ``edge_node_scatter_amd``.

Every function takes and returns numpy arrays in the operator's layouts:
dst (E,) int64, coupling (E,15) f32, radial (E,3,C) f32, grad_out (N,16,C) f32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zs_oracle.c")
_LIB = os.path.join(_HERE, "libzs_oracle.so")
_SRC_MT = os.path.join(_HERE, "zs_oracle_mt.c")
_LIB_MT = os.path.join(_HERE, "libzs_oracle_mt.so")

GCC_FLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-builtin-sqrt",
             "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Werror"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle library with gcc (no GPU involved)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def build_mt(force: bool = True) -> str:
    """Compile the K-thread variant (zs_oracle_mt.c, which includes
    zs_oracle.c) with gcc -fopenmp."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_MT))
    if force or not os.path.exists(_LIB_MT) or os.path.getmtime(_LIB_MT) < newest:
        tmp = _LIB_MT + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-fopenmp", _SRC_MT, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_MT)
    return _LIB_MT


_SIGS = {
    "zs_oracle_forward_f32": "PPPIIIP",
    "zs_oracle_forward_nodes_f32": "PPPIIIPIP",
    "zs_oracle_backward_f32": "PPPPIIIPP",
    "zs_oracle_backward_edges_f32": "PPPPIIIPIPP",
    "zs_oracle_forward_f64": "PPPIIIP",
    "zs_oracle_backward_f64": "PPPPIIIPP",
    "zs_oracle_csr": "PIIPPP",
    "zs_oracle_forward_norm_f32": "PPPPIIIPPP",
    "zs_oracle_backward_norm_f32": "PPPPPPIIIPPPP",
    "zs_oracle_forward_norm_f64": "PPPPIIIPP",
}


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _prep(dst, coupling, radial):
    dst = np.ascontiguousarray(dst, dtype=np.int64)
    coupling = np.ascontiguousarray(coupling, dtype=np.float32)
    radial = np.ascontiguousarray(radial, dtype=np.float32)
    E = dst.shape[0]
    if coupling.shape != (E, 15) or radial.ndim != 3 or radial.shape[:2] != (E, 3):
        raise ValueError("bad shapes")
    return dst, coupling, radial, E, radial.shape[2]


class OracleIndexError(IndexError):
    pass


def _check(rc):
    if rc == -3:
        raise OracleIndexError("destination index out of range")
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")


class Oracle:
    """The oracle functions bound to one compiled copy of zs_oracle.c."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        for name, sig in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p if ch == "P" else ctypes.c_int64 for ch in sig]
            fn.restype = ctypes.c_int
        self.lib = lib
        self.path = libpath

    def forward(self, coupling, radial, dst, n_nodes, dtype=np.float32):
        """out (N,16,C): fp32 sequential in edge order, or fp64 when dtype=float64."""
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        out = np.empty((n_nodes, 16, C), dtype=dtype)
        fn = self.lib.zs_oracle_forward_f64 if dtype == np.float64 else self.lib.zs_oracle_forward_f32
        _check(fn(_p(coupling), _p(radial), _p(dst), E, n_nodes, C, _p(out)))
        return out

    def forward_nodes(self, coupling, radial, dst, n_nodes, nodes):
        """out[nodes] only (len(nodes),16,C), same arithmetic as forward()."""
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        nodes = np.ascontiguousarray(nodes, dtype=np.int64)
        rows = np.empty((len(nodes), 16, C), dtype=np.float32)
        _check(self.lib.zs_oracle_forward_nodes_f32(_p(coupling), _p(radial), _p(dst), E, n_nodes,
                                                    C, _p(nodes), len(nodes), _p(rows)))
        return rows

    def backward(self, grad_out, coupling, radial, dst, dtype=np.float32):
        """(grad_coupling (E,15), grad_radial (E,3,C)); fp64 when dtype=float64."""
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
        N = grad_out.shape[0]
        if grad_out.shape != (N, 16, C):
            raise ValueError("bad grad_out shape")
        gc = np.empty((E, 15), dtype=dtype)
        gr = np.empty((E, 3, C), dtype=dtype)
        fn = self.lib.zs_oracle_backward_f64 if dtype == np.float64 else self.lib.zs_oracle_backward_f32
        _check(fn(_p(grad_out), _p(coupling), _p(radial), _p(dst), E, N, C, _p(gc), _p(gr)))
        return gc, gr

    def backward_edges(self, grad_out, coupling, radial, dst, edges):
        """Gradients of the sampled edges only: (len,15), (len,3,C)."""
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
        edges = np.ascontiguousarray(edges, dtype=np.int64)
        gc = np.empty((len(edges), 15), dtype=np.float32)
        gr = np.empty((len(edges), 3, C), dtype=np.float32)
        _check(self.lib.zs_oracle_backward_edges_f32(_p(grad_out), _p(coupling), _p(radial),
                                                     _p(dst), E, grad_out.shape[0], C, _p(edges),
                                                     len(edges), _p(gc), _p(gr)))
        return gc, gr

    def forward_norm(self, coupling, radial, env, dst, n_nodes, dtype=np.float32):
        """Scatter followed by the 1/sqrt(degree) normalisation.

        fp32: (y, out, norm); fp64: (y, norm)."""
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        env = np.ascontiguousarray(env, dtype=np.float32)
        if env.shape != (E,):
            raise ValueError("env must be (E,)")
        y = np.empty((n_nodes, 16, C), dtype=dtype)
        norm = np.empty(n_nodes, dtype=dtype)
        if dtype == np.float64:
            _check(self.lib.zs_oracle_forward_norm_f64(_p(coupling), _p(radial), _p(env), _p(dst),
                                                       E, n_nodes, C, _p(y), _p(norm)))
            return y, norm
        out = np.empty((n_nodes, 16, C), dtype=np.float32)
        _check(self.lib.zs_oracle_forward_norm_f32(_p(coupling), _p(radial), _p(env), _p(dst), E,
                                                   n_nodes, C, _p(y), _p(out), _p(norm)))
        return y, out, norm

    def backward_norm(self, grad_y, out, norm, coupling, radial, dst):
        """(grad_coupling, grad_radial, grad_env) of the normalised scatter (fp32)."""
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        grad_y = np.ascontiguousarray(grad_y, dtype=np.float32)
        out = np.ascontiguousarray(out, dtype=np.float32)
        norm = np.ascontiguousarray(norm, dtype=np.float32)
        N = grad_y.shape[0]
        gc = np.empty((E, 15), dtype=np.float32)
        gr = np.empty((E, 3, C), dtype=np.float32)
        ge = np.empty(E, dtype=np.float32)
        scratch = np.empty((N, 16, C), dtype=np.float32)
        _check(self.lib.zs_oracle_backward_norm_f32(_p(grad_y), _p(out), _p(norm), _p(coupling),
                                                    _p(radial), _p(dst), E, N, C, _p(gc), _p(gr),
                                                    _p(ge), _p(scratch)))
        return gc, gr, ge

    def csr(self, dst, n_nodes):
        """(rowptr (N+1,) int32, perm (E,) int32): stable counting sort by dst."""
        dst = np.ascontiguousarray(dst, dtype=np.int64)
        rowptr = np.empty(n_nodes + 1, dtype=np.int32)
        perm = np.empty(dst.shape[0], dtype=np.int32)
        cursor = np.empty(max(n_nodes, 1), dtype=np.int32)
        _check(self.lib.zs_oracle_csr(_p(dst), dst.shape[0], n_nodes, _p(rowptr), _p(perm),
                                      _p(cursor)))
        return rowptr, perm


_default = None


def get() -> Oracle:
    """The oracle built from the committed zs_oracle.c."""
    global _default
    if _default is None:
        build(force=False)
        _default = Oracle(_LIB)
    return _default


def forward(*a, **k):
    return get().forward(*a, **k)


def forward_nodes(*a, **k):
    return get().forward_nodes(*a, **k)


def backward(*a, **k):
    return get().backward(*a, **k)


def backward_edges(*a, **k):
    return get().backward_edges(*a, **k)


def csr(*a, **k):
    return get().csr(*a, **k)


def forward_norm(*a, **k):
    return get().forward_norm(*a, **k)


def backward_norm(*a, **k):
    return get().backward_norm(*a, **k)


class OracleMT:
    """The K-thread variant: node-blocked forward (each node's edges in
    increasing edge id, from the oracle's CSR) and edge-blocked backward,
    bitwise equal to the oracle's forward and backward."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        for name, sig in {"zs_oracle_mt_forward_f32": "PPPPIIPI",
                          "zs_oracle_mt_backward_f32": "PPPPIIIPPI"}.items():
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p if ch == "P" else ctypes.c_int64 for ch in sig]
            fn.restype = ctypes.c_int
        self.lib = lib

    def forward(self, coupling, radial, dst, n_nodes, threads, csr=None):
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        rowptr, perm = csr if csr is not None else get().csr(dst, n_nodes)
        rowptr = np.ascontiguousarray(rowptr, dtype=np.int32)
        perm = np.ascontiguousarray(perm, dtype=np.int32)
        out = np.empty((n_nodes, 16, C), dtype=np.float32)
        _check(self.lib.zs_oracle_mt_forward_f32(_p(coupling), _p(radial), _p(rowptr), _p(perm),
                                                 n_nodes, C, _p(out), threads))
        return out

    def backward(self, grad_out, coupling, radial, dst, threads):
        dst, coupling, radial, E, C = _prep(dst, coupling, radial)
        grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
        N = grad_out.shape[0]
        if grad_out.shape != (N, 16, C):
            raise ValueError("bad grad_out shape")
        gc = np.empty((E, 15), dtype=np.float32)
        gr = np.empty((E, 3, C), dtype=np.float32)
        _check(self.lib.zs_oracle_mt_backward_f32(_p(grad_out), _p(coupling), _p(radial), _p(dst),
                                                  E, N, C, _p(gc), _p(gr), threads))
        return gc, gr


_default_mt = None


def get_mt() -> OracleMT:
    """The K-thread variant built from the committed sources."""
    global _default_mt
    if _default_mt is None:
        build_mt(force=False)
        _default_mt = OracleMT(_LIB_MT)
    return _default_mt
