"""Python binding of libzs, the MI355X GIE zonal-scatter library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libzs.so`` (C ABI in ``include/zs.h``).  PyTorch supplies device
memory and the current HIP stream.  There is no CPU fallback: if the library
is missing or no GPU is present, these functions raise.

Functions carry the C ABI's names:

* ``zs_build_csr(dst, n_nodes)`` -> ``Csr(rowptr, perm, dst32, n_nodes, order)``
* ``zs_forward(coupling, radial, csr)`` -> out (N, 16, C)
* ``zs_backward(grad_out, coupling, radial, csr)`` -> (grad_coupling, grad_radial)
* ``zs_forward_normalized(coupling, radial, env, csr)`` -> (y, out, norm)
* ``zs_backward_normalized(grad_y, out, norm, coupling, radial, csr)``
  -> (grad_coupling, grad_radial, grad_env, grad_deg)

plus ``gie_zonal_scatter(coupling, radial, csr)``, an autograd function with
the operator boundary of deepmd-kit PR #6072 ("fused Triton zonal scatter for
the GIE head", section "Boundary and layout contract"): only fp32 is
accepted and no double backward is provided.  Unlike that boundary, strided
views of the edge inputs are read in place instead of being copied to
contiguous tensors (``zs_forward_strided`` / ``zs_backward_strided``).
``gie_zonal_scatter_normalized(coupling, radial, env, csr)`` adds the
inverse-square-root degree normalisation that follows the scatter on the same
page ("What", third bullet), with the envelope gradient it carries.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import NamedTuple

import torch  # load torch's HIP runtime first so libzs binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzs.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "zs.h")

ZS_OK = 0
ROWS, ZONAL, SLOTS = 16, 15, 3
MAX_CHANNELS = 1024

_lib = None


class ZsError(RuntimeError):
    """A libzs call returned a negative status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load libzs.so (built by edge_node_scatter_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        lib.zs_status_string.argtypes = [INT]
        lib.zs_status_string.restype = ctypes.c_char_p
        lib.zs_csr_workspace_bytes.argtypes = [I64, I64]
        lib.zs_csr_workspace_bytes.restype = SZ
        lib.zs_build_csr.argtypes = [P, I64, I64, P, P, P, P, P, SZ, P, P]
        lib.zs_build_csr.restype = INT
        lib.zs_build_csr_noalloc.argtypes = [P, I64, I64, P, P, P, P, P, P]
        lib.zs_build_csr_noalloc.restype = INT
        lib.zs_forward.argtypes = [P, P, P, P, P, I64, I64, I64, P, P]
        lib.zs_forward.restype = INT
        lib.zs_backward.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, P, P]
        lib.zs_backward.restype = INT
        lib.zs_forward_strided.argtypes = [P, I64, P, I64, I64, P, P, P, I64, I64, I64, P, P]
        lib.zs_forward_strided.restype = INT
        lib.zs_backward_strided.argtypes = [P, P, I64, P, I64, I64, P, P, P, I64, I64, I64, P, P,
                                            P]
        lib.zs_backward_strided.restype = INT
        lib.zs_forward_normalized.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, P, P, P]
        lib.zs_forward_normalized.restype = INT
        lib.zs_backward_normalized.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, P, P, P, P,
                                               P]
        lib.zs_backward_normalized.restype = INT
        _lib = lib
    return _lib


def declared_symbols() -> list[str]:
    """Function names declared in include/zs.h."""
    text = open(HEADER_PATH).read()
    return re.findall(r"^\w[\w\s\*]*?\b(zs_\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return load().zs_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != ZS_OK:
        raise ZsError(fn, status)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _call(dev: torch.device, fn, *args) -> int:
    """One library call with ``dev`` as the current device and its current
    stream as the last argument (the library launches on the current device
    and keeps its no-allocation scratch per device)."""
    with torch.cuda.device(dev):
        return fn(*args, torch.cuda.current_stream(dev).cuda_stream)


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype,
                contiguous: bool = True) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.contiguous() if contiguous else t


def _buffer(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype,
            device: torch.device) -> torch.Tensor:
    """A caller-supplied buffer the library reads as, or writes to, a dense
    array of ``shape``: anything else would let a kernel touch memory past it,
    so it is rejected rather than copied."""
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _csr_buffers(csr: "Csr", n_edges: int, device: torch.device) -> None:
    """The CSR arrays must hold N + 1 row offsets, E positions and (when
    present) N order entries."""
    _buffer(csr.rowptr, "csr.rowptr", (csr.n_nodes + 1,), torch.int32, device)
    _buffer(csr.perm, "csr.perm", (n_edges,), torch.int32, device)
    _buffer(csr.dst32, "csr.dst32", (n_edges,), torch.int32, device)
    if csr.order is not None:
        _buffer(csr.order, "csr.order", (csr.n_nodes,), torch.int32, device)


def _edge_views(coupling: torch.Tensor, radial: torch.Tensor):
    """Coupling (E,15) and radial (E,3,C) as views the strided entry points
    accept (unit-stride columns / channels, non-negative strides); anything
    else is copied to a contiguous tensor.  Returns the tensors and their
    (coupling edge, radial edge, radial slot) strides in floats."""
    if coupling.dim() != 2 or coupling.shape[1] != ZONAL:
        raise ValueError("coupling must be (E, 15)")
    if radial.dim() != 3 or radial.shape[1] != SLOTS or radial.shape[0] != coupling.shape[0]:
        raise ValueError("radial must be (E, 3, C) with the same E as coupling")
    if coupling.stride(1) != 1 or coupling.stride(0) < 0:
        coupling = coupling.contiguous()
    if radial.stride(2) != 1 or radial.stride(0) < 0 or radial.stride(1) < 0:
        radial = radial.contiguous()
    return coupling, radial, (coupling.stride(0), radial.stride(0), radial.stride(1))


def coupling_from_band(band: torch.Tensor, m0_offset: int = 15) -> torch.Tensor:
    """The zonal coupling (E, 15) as a view of a packed (E, 46) Wigner band.

    The band stores, per edge, three segments (the band page keeps three
    structural rows of each degree block): two of 15 entries and the m = 0
    segment of 16 entries (rows 0..15, row 0 being the l = 0 block).  The
    pages do not print the segment order; the default m0_offset = 15 reads
    them in increasing m (m = -1, 0, +1), so the coupling of rows 1..15 is
    band[:, 16:31].  The view is passed to the kernels without a copy.
    """
    if band.dim() != 2 or band.shape[1] != 3 * ROWS - 2:
        raise ValueError("band must be (E, 46)")
    return band[:, m0_offset + 1:m0_offset + 1 + ZONAL]


class Csr(NamedTuple):
    rowptr: torch.Tensor   # (N+1,) int32
    perm: torch.Tensor     # (E,) int32
    dst32: torch.Tensor    # (E,) int32
    n_nodes: int
    order: torch.Tensor | None = None   # (N,) int32 node order for the forward, or None


def zs_csr_workspace_bytes(n_edges: int, n_nodes: int) -> int:
    return int(load().zs_csr_workspace_bytes(n_edges, n_nodes))


def zs_build_csr(dst: torch.Tensor, n_nodes: int, workspace: torch.Tensor | None = None,
                 out: Csr | None = None, bad_flag: torch.Tensor | None = None,
                 order: bool = True) -> Csr:
    """Stable destination CSR of int64 ``dst``.

    Without ``bad_flag`` the call synchronizes the stream and raises ZsError
    (status ZS_ERR_INDEX) for a destination outside [0, n_nodes).  With a
    one-element int32 GPU tensor ``bad_flag`` it returns at once and the flag
    becomes nonzero, in stream order, if any destination was out of range.
    A new Csr carries the node order (nodes by decreasing degree) unless
    ``order`` is False; with ``out`` the order is written when out.order is
    a tensor.
    """
    dst = _dev_tensor(dst, "dst", torch.int64)
    E = dst.numel()
    dev = dst.device
    if out is None:
        out = Csr(torch.empty(n_nodes + 1, dtype=torch.int32, device=dev),
                  torch.empty(E, dtype=torch.int32, device=dev),
                  torch.empty(E, dtype=torch.int32, device=dev), n_nodes,
                  torch.empty(n_nodes, dtype=torch.int32, device=dev) if order else None)
    elif out.n_nodes != n_nodes:
        raise ValueError(f"out.n_nodes is {out.n_nodes}, expected {n_nodes}")
    _csr_buffers(out, E, dev)
    need = zs_csr_workspace_bytes(E, n_nodes)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _buffer(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    if bad_flag is not None:
        _buffer(bad_flag, "bad_flag", (1,), torch.int32, dev)
    _check("zs_build_csr", _call(
        dev, load().zs_build_csr, _ptr(dst), E, n_nodes, _ptr(out.rowptr), _ptr(out.perm),
        _ptr(out.dst32), _ptr(out.order), _ptr(workspace), workspace.numel(), _ptr(bad_flag)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def zs_build_csr_noalloc(dst: torch.Tensor, n_nodes: int, out: Csr,
                         bad_flag: torch.Tensor | None = None) -> Csr:
    """zs_build_csr with the library's fixed per-device scratch instead of a
    workspace: the call allocates nothing, so the output arrays must be
    passed in (``out``).  Raises ZsError (ZS_ERR_SCRATCH) when the sizes need
    more than NOALLOC_SCRATCH_BYTES of scratch.  Calls that overlap on one
    device share that scratch and must not run concurrently."""
    dst = _dev_tensor(dst, "dst", torch.int64, contiguous=False)
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    E = dst.numel()
    dev = dst.device
    if out.n_nodes != n_nodes:
        raise ValueError(f"out.n_nodes is {out.n_nodes}, expected {n_nodes}")
    _csr_buffers(out, E, dev)
    if bad_flag is not None:
        _buffer(bad_flag, "bad_flag", (1,), torch.int32, dev)
    _check("zs_build_csr_noalloc", _call(
        dev, load().zs_build_csr_noalloc, _ptr(dst), E, n_nodes, _ptr(out.rowptr),
        _ptr(out.perm), _ptr(out.dst32), _ptr(out.order), _ptr(bad_flag)))
    return out


def zs_forward(coupling: torch.Tensor, radial: torch.Tensor, csr: Csr,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """out (N, 16, C) fp32 with out[:, 0] = 0.  coupling and radial may be
    strided views (unit-stride last dimension); they are not copied."""
    coupling = _dev_tensor(coupling, "coupling", torch.float32, contiguous=False)
    radial = _dev_tensor(radial, "radial", torch.float32, contiguous=False)
    coupling, radial, (cs, re, rs) = _edge_views(coupling, radial)
    E, C = radial.shape[0], radial.shape[2]
    dev = radial.device
    if coupling.device != dev:
        raise ValueError("coupling and radial must be on the same device")
    _csr_buffers(csr, E, dev)
    if out is None:
        out = torch.empty((csr.n_nodes, ROWS, C), dtype=torch.float32, device=dev)
    else:
        _buffer(out, "out", (csr.n_nodes, ROWS, C), torch.float32, dev)
    if coupling.is_contiguous() and radial.is_contiguous():
        status = _call(dev, load().zs_forward, _ptr(coupling), _ptr(radial), _ptr(csr.rowptr),
                       _ptr(csr.perm), _ptr(csr.order), csr.n_nodes, E, C, _ptr(out))
    else:
        status = _call(dev, load().zs_forward_strided, _ptr(coupling), cs, _ptr(radial), re, rs,
                       _ptr(csr.rowptr), _ptr(csr.perm), _ptr(csr.order), csr.n_nodes, E, C,
                       _ptr(out))
    _check("zs_forward", status)
    return out


def zs_backward(grad_out: torch.Tensor, coupling: torch.Tensor, radial: torch.Tensor, csr: Csr,
                grad_coupling: torch.Tensor | None = None,
                grad_radial: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """(grad_coupling (E, 15), grad_radial (E, 3, C)) fp32, contiguous.
    coupling and radial may be strided views as in zs_forward."""
    grad_out = _dev_tensor(grad_out, "grad_out", torch.float32)
    coupling = _dev_tensor(coupling, "coupling", torch.float32, contiguous=False)
    radial = _dev_tensor(radial, "radial", torch.float32, contiguous=False)
    coupling, radial, (cs, re, rs) = _edge_views(coupling, radial)
    E, C = radial.shape[0], radial.shape[2]
    dev = radial.device
    _buffer(grad_out, "grad_out", (csr.n_nodes, ROWS, C), torch.float32, dev)
    if coupling.device != dev:
        raise ValueError("coupling and radial must be on the same device")
    _csr_buffers(csr, E, dev)
    if grad_coupling is None:
        grad_coupling = torch.empty((E, ZONAL), dtype=torch.float32, device=dev)
    else:
        _buffer(grad_coupling, "grad_coupling", (E, ZONAL), torch.float32, dev)
    if grad_radial is None:
        grad_radial = torch.empty((E, SLOTS, C), dtype=torch.float32, device=dev)
    else:
        _buffer(grad_radial, "grad_radial", (E, SLOTS, C), torch.float32, dev)
    if coupling.is_contiguous() and radial.is_contiguous():
        status = _call(dev, load().zs_backward, _ptr(grad_out), _ptr(coupling), _ptr(radial),
                       _ptr(csr.dst32), _ptr(csr.rowptr), _ptr(csr.perm), csr.n_nodes, E, C,
                       _ptr(grad_coupling), _ptr(grad_radial))
    else:
        status = _call(dev, load().zs_backward_strided, _ptr(grad_out), _ptr(coupling), cs,
                       _ptr(radial), re, rs, _ptr(csr.dst32), _ptr(csr.rowptr), _ptr(csr.perm),
                       csr.n_nodes, E, C, _ptr(grad_coupling), _ptr(grad_radial))
    _check("zs_backward", status)
    return grad_coupling, grad_radial


def _edge_inputs(coupling, radial):
    coupling = _dev_tensor(coupling, "coupling", torch.float32)
    radial = _dev_tensor(radial, "radial", torch.float32)
    if coupling.dim() != 2 or coupling.shape[1] != ZONAL:
        raise ValueError("coupling must be (E, 15)")
    if radial.dim() != 3 or radial.shape[1] != SLOTS or radial.shape[0] != coupling.shape[0]:
        raise ValueError("radial must be (E, 3, C) with the same E as coupling")
    return coupling, radial


def zs_forward_normalized(coupling: torch.Tensor, radial: torch.Tensor, env: torch.Tensor,
                          csr: Csr, keep_out: bool = True):
    """(y, out, norm): y = out * norm[:, None, None] with norm = deg^(-1/2)
    (0 where deg <= 0) and deg the per-node sum of ``env`` (E,).  ``out`` is
    the unnormalised scatter (None when ``keep_out`` is False).  Inputs are
    made contiguous."""
    coupling, radial = _edge_inputs(coupling, radial)
    env = _dev_tensor(env, "env", torch.float32)
    E, C = radial.shape[0], radial.shape[2]
    if env.shape != (E,):
        raise ValueError("env must be (E,)")
    dev = radial.device
    _buffer(env, "env", (E,), torch.float32, dev)
    _csr_buffers(csr, E, dev)
    y = torch.empty((csr.n_nodes, ROWS, C), dtype=torch.float32, device=dev)
    out = torch.empty_like(y) if keep_out else None
    norm = torch.empty(csr.n_nodes, dtype=torch.float32, device=dev)
    _check("zs_forward_normalized", _call(
        dev, load().zs_forward_normalized, _ptr(coupling), _ptr(radial), _ptr(env),
        _ptr(csr.rowptr), _ptr(csr.perm), _ptr(csr.order), csr.n_nodes, E, C, _ptr(y), _ptr(out),
        _ptr(norm)))
    return y, out, norm


def zs_backward_normalized(grad_y: torch.Tensor, out: torch.Tensor, norm: torch.Tensor,
                           coupling: torch.Tensor, radial: torch.Tensor, csr: Csr):
    """(grad_coupling (E, 15), grad_radial (E, 3, C), grad_env (E,),
    grad_deg (N,)) for y = zs_forward_normalized(...)[0]."""
    coupling, radial = _edge_inputs(coupling, radial)
    grad_y = _dev_tensor(grad_y, "grad_y", torch.float32)
    out = _dev_tensor(out, "out", torch.float32)
    norm = _dev_tensor(norm, "norm", torch.float32)
    E, C = radial.shape[0], radial.shape[2]
    N = csr.n_nodes
    if grad_y.shape != (N, ROWS, C) or out.shape != (N, ROWS, C) or norm.shape != (N,):
        raise ValueError("grad_y and out must be (N, 16, C), norm (N,)")
    dev = radial.device
    for name, t in (("grad_y", grad_y), ("out", out), ("norm", norm), ("coupling", coupling)):
        if t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
    _csr_buffers(csr, E, dev)
    gc = torch.empty((E, ZONAL), dtype=torch.float32, device=dev)
    gr = torch.empty((E, SLOTS, C), dtype=torch.float32, device=dev)
    ge = torch.empty(E, dtype=torch.float32, device=dev)
    gd = torch.empty(N, dtype=torch.float32, device=dev)
    _check("zs_backward_normalized", _call(
        dev, load().zs_backward_normalized, _ptr(grad_y), _ptr(out), _ptr(norm), _ptr(coupling),
        _ptr(radial), _ptr(csr.dst32), _ptr(csr.rowptr), _ptr(csr.perm), N, E, C, _ptr(gc),
        _ptr(gr), _ptr(ge), _ptr(gd)))
    return gc, gr, ge, gd


class _GieZonalScatter(torch.autograd.Function):
    @staticmethod
    def forward(ctx, coupling, radial, rowptr, perm, dst32, n_nodes, order):
        csr = Csr(rowptr, perm, dst32, n_nodes, order)
        ctx.save_for_backward(coupling, radial, rowptr, perm, dst32)
        ctx.n_nodes = n_nodes
        return zs_forward(coupling, radial, csr)

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, grad_out):
        coupling, radial, rowptr, perm, dst32 = ctx.saved_tensors
        csr = Csr(rowptr, perm, dst32, ctx.n_nodes)
        gc, gr = zs_backward(grad_out.contiguous(), coupling, radial, csr)
        return gc, gr, None, None, None, None, None


def gie_zonal_scatter(coupling: torch.Tensor, radial: torch.Tensor, csr: Csr) -> torch.Tensor:
    """Differentiable zonal scatter.  Strided views of coupling and radial (for
    example sliced radial features, or the coupling inside a packed Wigner
    band) are read in place; the gradients are contiguous tensors."""
    return _GieZonalScatter.apply(coupling, radial, csr.rowptr, csr.perm, csr.dst32, csr.n_nodes,
                                  csr.order)


class _GieZonalScatterNormalized(torch.autograd.Function):
    @staticmethod
    def forward(ctx, coupling, radial, env, rowptr, perm, dst32, n_nodes, order):
        csr = Csr(rowptr, perm, dst32, n_nodes, order)
        coupling, radial = coupling.contiguous(), radial.contiguous()
        y, out, norm = zs_forward_normalized(coupling, radial, env, csr)
        ctx.save_for_backward(coupling, radial, out, norm, rowptr, perm, dst32)
        ctx.n_nodes = n_nodes
        return y

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, grad_y):
        coupling, radial, out, norm, rowptr, perm, dst32 = ctx.saved_tensors
        csr = Csr(rowptr, perm, dst32, ctx.n_nodes)
        if grad_y is None:
            grad_y = torch.zeros_like(out)
        gc, gr, ge, _ = zs_backward_normalized(grad_y.contiguous(), out, norm, coupling, radial,
                                               csr)
        return gc, gr, ge, None, None, None, None, None


def gie_zonal_scatter_normalized(coupling: torch.Tensor, radial: torch.Tensor, env: torch.Tensor,
                                 csr: Csr) -> torch.Tensor:
    """Differentiable scatter followed by the degree normalisation:
    returns y = scatter * norm[:, None, None], norm = deg^(-1/2) with deg the
    per-node sum of ``env``.  Gradients flow to coupling, radial and env.
    The per-node factor itself is not returned here (a caller that used it
    downstream would expect a gradient through it, which this function does
    not carry); ``zs_forward_normalized`` returns it as a plain tensor."""
    return _GieZonalScatterNormalized.apply(coupling, radial, env, csr.rowptr, csr.perm,
                                            csr.dst32, csr.n_nodes, csr.order)
