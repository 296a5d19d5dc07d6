"""zs_build_csr_noalloc against zs_build_csr, through the C ABI on the GPU.

The no-allocation build runs the same kernels on the library's fixed
per-device scratch, so its CSR must be bitwise the one the workspace build
gives.  Two calls in a row, the second on a smaller frame, check that nothing
left in the shared scratch by the first call reaches the second's results.
"""
import numpy as np
import pytest
import torch

import edge_node_scatter_amd as zs
import synthetic

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zs.load()
    return torch.device("cuda:0")


def _empty_csr(n_nodes, n_edges, dev, fill):
    return zs.Csr(torch.full((n_nodes + 1,), fill, dtype=torch.int32, device=dev),
                  torch.full((n_edges,), fill, dtype=torch.int32, device=dev),
                  torch.full((n_edges,), fill, dtype=torch.int32, device=dev), n_nodes,
                  torch.full((n_nodes,), fill, dtype=torch.int32, device=dev))


def _same(a: zs.Csr, b: zs.Csr, what: str):
    for name in ("rowptr", "perm", "dst32", "order"):
        x, y = getattr(a, name).cpu().numpy(), getattr(b, name).cpu().numpy()
        assert np.array_equal(x, y), f"{what}: {name} differs"


def _frame(name, n_nodes, n_edges, seed):
    w = synthetic.custom(name, n_nodes, n_edges, 8, seed=seed)
    return w, synthetic.make_dst(w)


def test_noalloc_matches_workspace_build_twice(dev):
    """The 4096-node headline frame, then a smaller frame: both bitwise equal to
    the workspace build, with a synchronous and an asynchronous index check."""
    frames = [(synthetic.WORKLOADS["headline"], synthetic.make_dst(synthetic.WORKLOADS["headline"])),
              _frame("noalloc_small", 300, 20000, 77)]
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    for i, (w, dst_np) in enumerate(frames):
        N, E = w.n_nodes, w.n_edges
        say(f"[gpu] noalloc call {i}: N={N} E={E}")
        dst = torch.from_numpy(dst_np).to(dev)
        ref = zs.zs_build_csr(dst, N)
        got = zs.zs_build_csr_noalloc(dst, N, _empty_csr(N, E, dev, -7))
        torch.cuda.synchronize()
        _same(got, ref, f"call {i} (synchronous check)")
        flag.fill_(5)
        got2 = zs.zs_build_csr_noalloc(dst, N, _empty_csr(N, E, dev, -9), bad_flag=flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        _same(got2, ref, f"call {i} (asynchronous check)")


def test_noalloc_large_frame_then_tiny(dev):
    """The 16384-node frame (20.5 MiB of scratch), then the 64-node frame."""
    for name in ("large", "tiny"):
        w = synthetic.WORKLOADS[name]
        N, E = w.n_nodes, w.n_edges
        say(f"[gpu] noalloc {name}: N={N} E={E}")
        dst = torch.from_numpy(synthetic.make_dst(w)).to(dev)
        ref = zs.zs_build_csr(dst, N)
        got = zs.zs_build_csr_noalloc(dst, N, _empty_csr(N, E, dev, -3))
        torch.cuda.synchronize()
        _same(got, ref, name)


def test_noalloc_index_error_and_empty(dev):
    """An out-of-range destination is reported (ZS_ERR_INDEX, or the flag) as by
    zs_build_csr; no edges gives an all-zero rowptr; sizes past the scratch are
    refused before any work."""
    say("[gpu] noalloc: out-of-range destination, empty frame, oversized frame")
    N = 50
    dst_np = np.random.default_rng(5).integers(0, N, size=4000).astype(np.int64)
    dst_np[1234] = N
    dst = torch.from_numpy(dst_np).to(dev)
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_build_csr_noalloc(dst, N, _empty_csr(N, 4000, dev, 0))
    assert ei.value.status == -3
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    zs.zs_build_csr_noalloc(dst, N, _empty_csr(N, 4000, dev, 0), bad_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) != 0
    empty = zs.zs_build_csr_noalloc(torch.empty(0, dtype=torch.int64, device=dev), N,
                                    _empty_csr(N, 0, dev, 9))
    torch.cuda.synchronize()
    assert np.array_equal(empty.rowptr.cpu().numpy(), np.zeros(N + 1, np.int32))
    big_e = 5_000_000
    big = torch.zeros(big_e, dtype=torch.int64, device=dev)
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_build_csr_noalloc(big, 4096, _empty_csr(4096, big_e, dev, 0))
    assert ei.value.status == -8
    # a valid call after the refusals still matches the workspace build
    w, d = _frame("noalloc_after", 128, 9000, 13)
    dst = torch.from_numpy(d).to(dev)
    ref = zs.zs_build_csr(dst, 128)
    got = zs.zs_build_csr_noalloc(dst, 128, _empty_csr(128, 9000, dev, -1))
    torch.cuda.synchronize()
    _same(got, ref, "after refusals")
