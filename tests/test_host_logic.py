"""Host-side logic (CPU only): the seeded workload recipes and bench.py's
bookkeeping (algorithmic bytes, counter summaries, the one-GPU contract)."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", ["tiny", "n1000", "headline", "skewed"])
def test_workload_sizes_and_ranges(name):
    w = synthetic.WORKLOADS[name]
    x = synthetic.make_inputs(w)
    E, N, C = w.n_edges, w.n_nodes, w.channels
    assert x["dst"].shape == (E,) and x["dst"].dtype == np.int64
    assert x["dst"].min() >= 0 and x["dst"].max() < N
    assert x["coupling"].shape == (E, 15) and x["coupling"].dtype == np.float32
    assert x["radial"].shape == (E, 3, C) and x["radial"].dtype == np.float32
    assert x["grad_out"].shape == (N, 16, C)
    assert x["env"].shape == (E,) and np.all((x["env"] >= 0) & (x["env"] < 1))
    assert np.all(np.abs(x["coupling"]) <= 1.0)
    if w.envelope:   # coupling = U(-1, 1) * env, so |coupling| <= env
        assert np.all(np.abs(x["coupling"]) <= x["env"][:, None] + 1e-7)


def test_headline_degrees_near_constant():
    """647170 = 4096 * 158 + 2: all nodes of degree 158 but two of 159."""
    w = synthetic.WORKLOADS["headline"]
    deg = np.bincount(synthetic.make_dst(w), minlength=w.n_nodes)
    assert deg.sum() == 647170
    assert sorted(set(deg.tolist())) == [158, 159] and np.count_nonzero(deg == 159) == 2


def test_skewed_degrees():
    w = synthetic.WORKLOADS["skewed"]
    deg = np.bincount(synthetic.make_dst(w), minlength=w.n_nodes)
    assert deg.sum() == w.n_edges
    assert np.count_nonzero(deg == 0) >= 64
    live = np.sort(deg[deg > 0])
    lo, hi = live[: len(live) // 2], live[len(live) // 2:]
    assert 30 < lo.mean() < 50 and 250 < hi.mean() < 300   # Poisson(40) / Poisson(275) halves


def test_edge_order_is_shuffled():
    """Destinations are not grouped: consecutive edges rarely share a node."""
    d = synthetic.make_dst(synthetic.WORKLOADS["headline"])
    assert np.mean(d[1:] == d[:-1]) < 0.01


def test_inputs_deterministic_and_streams_independent():
    w = synthetic.WORKLOADS["tiny"]
    a, b = synthetic.make_inputs(w), synthetic.make_inputs(w)
    for k in ("dst", "coupling", "radial", "grad_out", "env"):
        assert np.array_equal(a[k], b[k]), k
    # a different channel count changes radial but no other tensor's values
    w2 = synthetic.custom("tiny_c8", w.n_nodes, w.n_edges, 8, w.seed, w.dst_kind, w.envelope)
    c = synthetic.make_inputs(w2)
    for k in ("dst", "coupling", "env"):
        assert np.array_equal(a[k], c[k]), k


def test_algorithmic_bytes_match_the_published_arithmetic():
    """Headline shape: forward 298.3 MB, backward 585.7 MB, together 884.0 MB;
    at 8 TB/s that is 110.5 us, and 60 % of peak is at most 184.2 us."""
    nb = bench.algorithmic_bytes(647170, 4096, 32)
    assert round(nb["fwd"] / 1e6, 1) == 298.3
    assert round(nb["bwd"] / 1e6, 1) == 585.7
    total = nb["fwd"] + nb["bwd"]
    assert round(total / 1e6, 1) == 884.0
    assert round(total / 8e12 * 1e6, 1) == 110.5
    assert round(total / (0.6 * 8e12) * 1e6, 1) == 184.2
    large = bench.algorithmic_bytes(2600000, 16384, 64)
    assert round((large["fwd"] + large["bwd"]) / 1e6, 1) == 6613.5
    nn = bench.algorithmic_bytes_normalized(647170, 4096, 32)
    assert nn["fwd"] - nb["fwd"] == 4 * 647170 + 4096 * (16 * 32 * 4 + 4)
    assert nn["bwd"] - nb["bwd"] == 4096 * (15 * 32 * 4 + 8) + 8 * 647170


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_source_hash_ignores_comments_only():
    """Counter data stays valid across comment and whitespace edits of a
    kernel source, and not across any change of its code."""
    src = "int f(int a) {  // adds one\n    return a + 1; /* the\n  sum */ }\n"
    same = "// header\nint f(int a) {\n  return a + 1;\n}\n"
    assert bench._code_only(src) == bench._code_only(same)
    for changed in ("int f(int a) { return a + 2; }", "int f(int b) { return b + 1; }",
                    "int f(int a) { return a - 1; }"):
        assert bench._code_only(changed) != bench._code_only(src)


def test_write_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kib = bench.COPY_CALIBRATION_BYTES / 1024
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    bwd = "void zs::(anonymous namespace)::zs_bwd_staged_kernel<8, 4, true>(float const*)"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", kib / 2),   # reads half
                                       (bwd, 1000.0), (bwd, 1200.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", kib), (bwd, 500.0)])
    out = bench.write_traffic(str(fetch), str(write))
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    k = out["kernels"]["zs_bwd_staged_kernel"]
    assert k["fetch_bytes"] == round(1100.0 * 1024 * 2.0)
    assert k["hbm_bytes_per_launch"] == round(1100.0 * 1024 * 2.0 + 500.0 * 1024)
    assert k["source_hash"] == bench.kernel_source_hash("bwd")
    assert bench.load_traffic("zs_bwd_staged_kernel") == k["hbm_bytes_per_launch"]
    # a record taken on other sources is not reported
    k["source_hash"] = "0" * 16
    with open(bench.TRAFFIC_FILE, "w") as f:
        json.dump(out, f)
    assert bench.load_traffic("zs_bwd_staged_kernel") is None


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_tiled_radial_rows_match_the_materialised_tiling():
    """Rows picked by formula equal the rows of the flat tiled array, which is
    how the device builds it (a 1-D repeat of the pool, then a view)."""
    w = synthetic.custom("tiled", 7, 50, 5, seed=3)
    pool = synthetic.radial_pool(w, length=101)        # prime, shorter than E * 3 * C
    flat = np.tile(pool, -(-50 * 3 * 5 // 101))[: 50 * 3 * 5].reshape(50, 3, 5)
    edges = np.array([0, 1, 6, 7, 33, 49])
    assert np.array_equal(synthetic.tiled_radial_rows(pool, edges, 5), flat[edges])
    big = synthetic.radial_pool(w)
    assert big.shape == (synthetic.RADIAL_POOL_LEN,) and big.dtype == np.float32
    assert abs(float(big.mean())) < 1e-3 and abs(float(big.std()) - 1.0) < 1e-3
    assert (2 ** 32) % synthetic.RADIAL_POOL_LEN != 0


def test_forward_rows_of_a_node_subset_need_only_their_edges():
    """The sampled parity check at sizes past 2^31 elements runs the oracle on
    just the sampled nodes' edges (increasing edge id, destinations renumbered);
    on a small frame that equals the full oracle's rows bit for bit, and the
    per-edge backward of a subset equals the full backward's rows."""
    import oracle
    w = synthetic.custom("subset", 40, 3000, 8, seed=11, envelope=True)
    x = synthetic.make_inputs(w)
    full = oracle.forward(x["coupling"], x["radial"], x["dst"], 40)
    nodes = np.array([0, 3, 17, 39])
    sub = np.flatnonzero(np.isin(x["dst"], nodes))
    part = oracle.forward(x["coupling"][sub], x["radial"][sub],
                          np.searchsorted(nodes, x["dst"][sub]), len(nodes))
    assert np.array_equal(part.view(np.uint32), full[nodes].view(np.uint32))
    gc, gr = oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
    edges = np.array([0, 5, 2999])
    gc_s, gr_s = oracle.backward(x["grad_out"], x["coupling"][edges], x["radial"][edges],
                                 x["dst"][edges])
    assert np.array_equal(gc_s.view(np.uint32), gc[edges].view(np.uint32))
    assert np.array_equal(gr_s.view(np.uint32), gr[edges].view(np.uint32))


def test_grouped_headline_is_the_headline_frame_sorted():
    """Same degrees and per-edge values as the headline frame, edges in
    destination order (so its CSR permutation is the identity)."""
    a = synthetic.make_inputs("headline", with_grad=False)
    b = synthetic.make_inputs("headline_grouped", with_grad=False)
    assert np.array_equal(np.bincount(a["dst"], minlength=4096), np.bincount(b["dst"], minlength=4096))
    assert np.all(np.diff(b["dst"]) >= 0)
    for k in ("coupling", "radial", "env"):
        assert np.array_equal(a[k], b[k]), k


def test_protocol_takes_the_median_of_process_medians(monkeypatch):
    """bench.py --processes N: each child reports its medians; the parent
    reports, per quantity, the median over the children."""
    import argparse
    import types
    outs = iter([
        {"flushed": {"build_us": 40, "fwd_us": 65, "bwd_us": 140, "fwd_bwd_us": 205},
         "flushed_fill": {"build_us": 40, "fwd_us": 66, "bwd_us": 141, "fwd_bwd_us": 207},
         "warm": {"build_us": 36, "fwd_us": 57, "bwd_us": 119, "fwd_bwd_us": 176}},
        {"flushed": {"build_us": 42, "fwd_us": 64, "bwd_us": 150, "fwd_bwd_us": 214},
         "flushed_fill": {"build_us": 42, "fwd_us": 65, "bwd_us": 151, "fwd_bwd_us": 216},
         "warm": {"build_us": 37, "fwd_us": 58, "bwd_us": 120, "fwd_bwd_us": 178}},
        {"flushed": {"build_us": 41, "fwd_us": 66, "bwd_us": 145, "fwd_bwd_us": 211},
         "flushed_fill": {"build_us": 41, "fwd_us": 67, "bwd_us": 146, "fwd_bwd_us": 213},
         "warm": {"build_us": 35, "fwd_us": 56, "bwd_us": 118, "fwd_bwd_us": 174}},
    ])
    calls = []

    def fake_run(cmd, **kw):
        calls.append(cmd)
        return types.SimpleNamespace(returncode=0, stdout="log line\n" + json.dumps(next(outs)),
                                     stderr="")

    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    args = argparse.Namespace(processes=3, workload="headline", inputs="contiguous", channels=None)
    nb = bench.algorithmic_bytes(647170, 4096, 32)
    rep = bench.run_protocol(args, nb)
    assert len(calls) == 3 and all("--protocol-child" in c for c in calls)
    assert rep["flushed"] == {"build_us": 41, "fwd_us": 65, "bwd_us": 145, "fwd_bwd_us": 211,
                              "gbs": round((nb["fwd"] + nb["bwd"]) / 211e-6 / 1e9, 1),
                              "hbm_frac": round((nb["fwd"] + nb["bwd"]) / 211e-6 / 1e9 / 8000, 4)}
    assert rep["warm"]["fwd_bwd_us"] == 176 and rep["warm"]["build_us"] == 36
    assert rep["per_process_fwd_bwd_us"]["flushed"] == [205, 214, 211]
    assert rep["flushed_fill"]["fwd_bwd_us"] == 213


def test_pages_context_is_the_pages_timings_over_the_same_bytes():
    """The RTX 5090 figures ride beside the result as context: 0.2 ms forward +
    0.5 ms backward over the same algorithmic bytes (884.0 MB at the headline
    shape) is ~1.26 TB/s, and the time ratio is 700 us over ours."""
    nb = bench.algorithmic_bytes(647170, 4096, 32)
    ctx = bench.pages_context(175.0, nb)
    assert ctx["fwd_bwd_us"] == 700.0
    assert ctx["algorithmic_gbs"] == pytest.approx(1262.9, abs=0.1)
    assert ctx["time_ratio"] == 4.0


def test_summarize_counters_means_per_kernel(tmp_path):
    """Counter summaries average each counter over a kernel's dispatches and
    keep only the library's kernels."""
    rows = [("void zs::(anonymous namespace)::zs_bwd_staged_kernel<8, 4, true>(float const*)",
             "SQ_WAVES", 16384), ("void zs::(anonymous namespace)::zs_bwd_staged_kernel<8, 4, "
                                  "true>(float const*)", "SQ_WAVES", 16386),
            ("at::native::fill", "SQ_WAVES", 5)]
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    got = bench.summarize_counters([str(p)])
    assert list(got) == ["zs::zs_bwd_staged_kernel<8, 4, true>"]
    assert got["zs::zs_bwd_staged_kernel<8, 4, true>"]["SQ_WAVES"] == {"mean": 16385.0,
                                                                     "dispatches": 2}


def test_kernel_roofline_figures():
    """Per-kernel figures: algorithmic bytes over the mean launch time, as a
    fraction of 8 TB/s; no counter figure away from the headline frame."""
    r = bench.kernel_roofline("zs_fwd_staged_kernel", 298337156, 57.0, headline=False)
    assert r["achieved_gbs"] == pytest.approx(5234.0, abs=0.1)
    assert r["frac"] == pytest.approx(0.6543, abs=1e-4)
    assert r["traffic"] is None and r["traffic_over_algorithmic"] is None
