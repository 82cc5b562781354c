"""Summarise a rocprofv3 results database (rocpd SQLite) per kernel:
calls, total/average/min/max duration.  Reads only the database file.

    python -m sparse_moe_layer_03_amd.rocpd_stats path/to/results.db [--skip N | --calls A:B] [name-substring]

--skip N leaves out the first N calls of every kernel (in start order), e.g.
the warm-up steps of a bench run, so that the averages cover the timed steps.
--calls A:B keeps calls A..B-1 of every kernel (0-based, in start order), e.g.
one pass of a bench run.
"""
import sqlite3
import sys


def main(path, filt=None, skip=0, stop=None):
    cur = sqlite3.connect(path).cursor()
    data = {}
    for name, start, dur, gx, wx, v, ag, lds in cur.execute(
            "select name, start, duration, grid_x, workgroup_x, vgpr_count, accum_vgpr_count, "
            "lds_size from kernels order by start"):
        d = data.setdefault(name, {"durs": [], "meta": (gx, wx, v, ag, lds)})
        d["durs"].append(dur)
    rows = []
    for name, d in data.items():
        durs = d["durs"][skip:stop]
        if not durs:
            continue
        rows.append((name, len(durs), sum(durs), sum(durs) / len(durs), min(durs), max(durs),
                     *d["meta"]))
    rows.sort(key=lambda r: -r[2])
    tot = sum(r[2] for r in rows) or 1
    print(f"{'kernel':<70} {'calls':>6} {'total_us':>10} {'avg_us':>9} {'min_us':>9} "
          f"{'max_us':>9} {'pct':>6}  grid wg vgpr agpr lds")
    for n, c, s, a, mn, mx, gx, wx, v, ag, lds in rows:
        if filt and filt not in n:
            continue
        print(f"{n[:70]:<70} {c:>6} {s/1e3:>10.1f} {a/1e3:>9.2f} {mn/1e3:>9.2f} {mx/1e3:>9.2f} "
              f"{100*s/tot:>6.1f}  {gx} {wx} {v} {ag} {lds}")


if __name__ == "__main__":
    args = sys.argv[1:]
    skip, stop = 0, None
    if "--skip" in args:
        i = args.index("--skip")
        skip = int(args[i + 1])
        del args[i:i + 2]
    if "--calls" in args:
        i = args.index("--calls")
        a, b = args[i + 1].split(":")
        skip, stop = int(a), int(b)
        del args[i:i + 2]
    main(args[0], args[1] if len(args) > 1 else None, skip, stop)
