"""bench.py's host-side pieces: byte accounting, the counter-summary guard, the one-GPU rule."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes():
    # n inputs + residual read, residual_out + out written, weight read once
    assert bench.algorithmic_bytes(8, 4096, 7168) == 2 * 11 * 4096 * 7168 + 2 * 7168 == 645937152
    assert bench.algorithmic_bytes(4, 8, 4096) == 466944


def test_traffic_reported_only_for_the_profiled_sources(monkeypatch):
    t = bench.measured_traffic()
    if t is not None:  # the committed summary matches the current kernel sources
        assert abs(t / bench.algorithmic_bytes(8, 4096, 7168) - 1) < 0.01
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "single MI355X" in r.stderr


def test_parity_rows_stay_in_range():
    # m = 1 once sampled row 1 of a one-row tensor (an out-of-bounds device gather)
    for m in (1, 2, 3, 4096):
        rows = bench.parity_rows(m)
        assert rows.min() == 0 and rows.max() == m - 1 and len(set(rows.tolist())) == len(rows)
    assert bench.parity_rows(1).tolist() == [0]


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    copies = []
    for i, path in enumerate(bench.KERNEL_SOURCES):
        dst = tmp_path / f"src{i}"
        dst.write_text(open(path).read())
        copies.append(str(dst))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", copies)
    base = bench.kernel_source_digest()
    with open(copies[0], "a") as f:
        f.write("\n// a comment\n/* another\n   comment */\n")
    assert bench.kernel_source_digest() == base
    with open(copies[0], "a") as f:
        f.write("\nstatic int extra_symbol = 1;\n")
    assert bench.kernel_source_digest() != base


def test_oracle_timing_on_threads_matches_single_thread():
    import oracle
    from all_reduce_residual_way_amd import synth
    prob = synth.make_problem(4, 37, 64, seed=5)
    got = bench.time_oracle(oracle.default(), prob, prob.eps, 10_000)
    assert got["threads_match_single"]
    assert got["oracle_1t_runs"] == 5 and 1 <= got["oracle_threads"] <= 16
    assert got["oracle_1t_ms"] > 0 and got["oracle_threads_ms"] > 0
    assert bench.oracle_runs(2e9) == 1 and bench.oracle_runs(5e8) == 5


def test_host_info_names_cpus():
    info = bench.host_info()
    assert info["host_cpus"] >= 1 and 1 <= info["affinity_cpus"] <= info["host_cpus"]
    assert bench.host_threads() == min(16, info["affinity_cpus"])


def test_cold_copies_exceed_the_cache():
    assert bench.cold_copies(100 << 20) == 1          # timed warm
    for fp in (200 << 20, 646 << 20, 1 << 30, 3 << 30):
        c = bench.cold_copies(fp)
        assert c * fp >= (1 << 30) or c == bench.MAX_SETS
    # between two calls on one set the other sets write at least twice the 256 MB cache
    for n, m, hidden in ((8, 4096, 7168), (8, 2048, 7168), (4, 4096, 7168), (8, 8192, 8192),
                         (8, 1024, 7168), (8, 16384, 2880)):
        fp, w = 2 * (n + 3) * m * hidden, bench.outputs_bytes(m, hidden)
        c = bench.cold_copies(fp, w)
        assert c * fp >= (1 << 30) and (c - 1) * w >= (512 << 20) and c <= bench.MAX_SETS
    assert bench.cold_copies(646 << 20, bench.outputs_bytes(4096, 7168)) == 6  # the bench shape
    # the metric's other rows (N=8, hidden 7168): 11 sets at m = 2048, 4 at m = 8192
    for m, sets in ((2048, 11), (4096, 6), (8192, 4)):
        fp = 2 * 11 * m * 7168
        assert bench.cold_copies(fp, bench.outputs_bytes(m, 7168)) == sets, m


def test_load_source_shapes_straddle_the_stream_rule():
    # the shapes that compare load policies: every one but the largest reads at most 128 MiB and so
    # takes ordinary loads automatically; the plan says so without touching a GPU
    import all_reduce_residual_way_amd as fa
    streams = {}
    for n, m, hidden in bench.LOAD_SOURCE_SHAPES:
        read = 2 * (n + 1) * m * hidden
        streams[(n, m, hidden)] = bool(fa.describe_launch(n, m, hidden, 1)["kernels"][0]["streaming"])
        assert streams[(n, m, hidden)] == (read > (128 << 20))
    assert sum(streams.values()) == 1 and streams[(8, 4096, 7168)]
