"""Host-side checks of the measurement helpers (no GPU): the source hash that
decides whether the bench reports committed HBM-traffic counters, the parser
of the committed traffic summaries, and the per-kernel summary of a rocprofv3
results database."""
import contextlib
import glob
import io
import os
import re
import sqlite3

from sparse_moe_layer_03_amd import rocpd_stats
from sparse_moe_layer_03_amd import traffic as TR

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_source_hash_ignores_comments_and_blank_lines_only(tmp_path):
    a = tmp_path / "k.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // add one\n}\n")
    h0 = TR.source_hash([str(a)])
    a.write_text("// a new header comment\n\nint f(int x) {\n  return x + 1;  // plus one\n}\n")
    assert TR.source_hash([str(a)]) == h0
    a.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert TR.source_hash([str(a)]) != h0


def test_source_hash_depends_on_file_names_not_argument_order(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    a.write_text("int a;\n")
    b.write_text("int b;\n")
    assert TR.source_hash([str(a), str(b)]) == TR.source_hash([str(b), str(a)])
    c = tmp_path / "c.hip"
    c.write_text("int a;\n")
    assert TR.source_hash([str(c), str(b)]) != TR.source_hash([str(a), str(b)])


def test_committed_traffic_summaries_parse():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt")))
    assert any("traffic_gate_up_" in p for p in paths)
    assert any("traffic_down_" in p for p in paths)
    for p in paths:
        s = TR.read_summary(p)
        assert re.fullmatch(r"[0-9a-f]{16}", s["source_hash"]), p
        assert float(s["traffic_bytes"]) > 0, p
        assert s["sources"] and all(os.path.exists(os.path.join(ROOT, q)) for q in s["sources"]), p


def test_bench_traffic_follows_the_summary_and_its_source_hash():
    import bench

    for kernel in ("gate_up", "down"):
        for p in sorted(glob.glob(os.path.join(ROOT, "profiles", f"traffic_{kernel}_*.txt"))):
            w = os.path.basename(p)[len(f"traffic_{kernel}_"):-len(".txt")]
            s = TR.read_summary(p)
            fresh = TR.source_hash([os.path.join(ROOT, q) for q in s["sources"]]) == s["source_hash"]
            got = bench.measured_traffic(w, kernel)
            assert got == (float(s["traffic_bytes"]) if fresh else None), p
    assert bench.measured_traffic("no_such_workload", "down") is None


def _db(path, durations):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, duration integer, grid_x integer, "
                "workgroup_x integer, vgpr_count integer, accum_vgpr_count integer, lds_size integer)")
    for i, (name, d) in enumerate(durations):
        con.execute("insert into kernels values (?, ?, ?, 256, 256, 32, 0, 0)", (name, i, d))
    con.commit()
    con.close()


def _avg(out, name):
    for ln in out.splitlines():
        if ln.startswith(name):
            return float(ln.split()[-9])  # avg_us column
    raise AssertionError(out)


def test_rocpd_stats_skip_and_call_range(tmp_path):
    db = str(tmp_path / "r.db")
    # kernel A: calls of 1, 2, 3, 4, 5 us (in start order); kernel B interleaved
    rows = []
    for i in range(5):
        rows.append(("kernA", (i + 1) * 1000))
        rows.append(("kernB", 7000))
    _db(db, rows)
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        rocpd_stats.main(db, None, 2)
    assert _avg(buf.getvalue(), "kernA") == 4.0  # calls 2..4: 3, 4, 5 us
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        rocpd_stats.main(db, "kernA", 1, 3)
    out = buf.getvalue()
    assert _avg(out, "kernA") == 2.5  # calls 1..2: 2, 3 us
    assert "kernB" not in out


def _counter_csv(path, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, counter, value) in enumerate(rows):
            f.write(f'{i},"{name}",{counter},{value}\n')


def test_traffic_summary_sums_the_kernels_of_one_call(tmp_path):
    # one call launches two kernels (320-row and 256-row tiles): the figure
    # per call is the sum of the two kernels' per-dispatch medians, scaled by
    # the copy probe's counter KiB per KiB moved
    a, b = "void grouped_gemm_big_kernel<1, 4, 1>(GemmArgs)", "void grouped_gemm_big_kernel<1, 4, 0>(GemmArgs)"
    kf, kw = str(tmp_path / "kf.csv"), str(tmp_path / "kw.csv")
    cf, cw = str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv")
    _counter_csv(kf, [(a, "FETCH_SIZE", 100.0), (b, "FETCH_SIZE", 50.0), (a, "FETCH_SIZE", 300.0),
                      (b, "FETCH_SIZE", 70.0), (a, "FETCH_SIZE", 200.0), (b, "FETCH_SIZE", 60.0)])
    _counter_csv(kw, [(a, "WRITE_SIZE", 10.0), (b, "WRITE_SIZE", 20.0)])
    kib = TR.COPY_BYTES / 1024.0
    _counter_csv(cf, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 0.5 * kib)])
    _counter_csv(cw, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1.0 * kib)])
    src = tmp_path / "k.hip"
    src.write_text("int k;\n")
    out = str(tmp_path / "t.txt")
    args = ["summarize", out, "--kernel-fetch", kf, "--kernel-write", kw, "--copy-fetch", cf,
            "--copy-write", cw, "--kernel-regex", "grouped_gemm_big_kernel<1,",
            "--copy-regex", "copyBuffer", "--source", str(src), "--command", "test"]
    with contextlib.redirect_stdout(io.StringIO()):
        TR.main(args)
    s = TR.read_summary(out)
    # medians 200 + 60 KiB fetched at 0.5 counter KiB per KiB -> 520 KiB read
    assert float(s["traffic_fetch_bytes"]) == (200.0 + 60.0) * 1024 / 0.5
    assert float(s["traffic_write_bytes"]) == (10.0 + 20.0) * 1024
    assert float(s["traffic_bytes"]) == 520 * 1024 + 30 * 1024
    assert s["source_hash"] == TR.source_hash([str(src)])


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU only" in r.stderr
