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
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_gate_up_*.txt")))
    assert paths
    for p in paths:
        s = TR.read_summary(p)
        assert re.fullmatch(r"[0-9a-f]{16}", s["source_hash"]), p
        assert float(s["traffic_bytes"]) > 0, p
        assert s["sources"] and all(os.path.exists(os.path.join(ROOT, q)) for q in s["sources"]), p


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
