"""Summarise a rocprofv3 results database (rocpd SQLite) per kernel:
calls, total/average/min/max duration.  Reads only the database file.

    python -m sparse_moe_layer_03_amd.rocpd_stats path/to/results.db [name-substring]
"""
import sqlite3
import sys


def main(path, filt=None):
    cur = sqlite3.connect(path).cursor()
    rows = cur.execute(
        "select name, count(*), sum(duration), avg(duration), min(duration), max(duration), "
        "max(grid_x), max(workgroup_x), max(vgpr_count), max(accum_vgpr_count), max(lds_size) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    tot = sum(r[2] for r in rows)
    print(f"{'kernel':<70} {'calls':>6} {'total_us':>10} {'avg_us':>9} {'min_us':>9} "
          f"{'max_us':>9} {'pct':>6}  grid wg vgpr agpr lds")
    for n, c, s, a, mn, mx, gx, wx, v, ag, lds in rows:
        if filt and filt not in n:
            continue
        print(f"{n[:70]:<70} {c:>6} {s/1e3:>10.1f} {a/1e3:>9.2f} {mn/1e3:>9.2f} {mx/1e3:>9.2f} "
              f"{100*s/tot:>6.1f}  {gx} {wx} {v} {ag} {lds}")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else None)
