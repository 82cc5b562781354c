"""MFMA utilisation of a kernel from one rocprofv3 --pmc pass.

    python -m sparse_moe_layer_03_amd.counters summarize OUT.txt --csv K.csv \\
        --kernel-regex REGEX --title "..." --command "..." \\
        [--alg-flops F] [--source FILE ...]

Reads a rocprofv3 counter_collection CSV holding SQ_VALU_MFMA_BUSY_CYCLES,
SQ_BUSY_CYCLES, SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_INSTS_MFMA,
SQ_INSTS_VALU_MFMA_MOPS_BF16 and GRBM_GUI_ACTIVE for the dispatches of one
kernel and writes a text summary: per-dispatch medians and the derived
figures (rocprofv3's own MfmaUtil definition: MFMA busy cycles over the
GUI-active cycles per XCD times the chip's 1024 SIMDs; executed bf16 flops =
MOPS x 512; the effective shader clock those cycles imply over the dispatch
duration).  --alg-flops gives the kernel's algorithmic flops per dispatch
(e.g. 4 A d_model d_ff for the gate/up GEMM) for the padding ratio.
"""

from __future__ import annotations

import argparse
import csv
import os
import re
import statistics

from sparse_moe_layer_03_amd import traffic as TR

COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY",
            "SQ_WAIT_INST_ANY", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
            "GRBM_GUI_ACTIVE")
XCDS = 8
SIMDS = 1024
PEAK_BF16 = 2.5e15


def read(path, regex):
    """{counter: [value per dispatch]}, [duration ns per dispatch], kernel name."""
    rx = re.compile(regex)
    per = {}
    durs = {}
    name = None
    with open(path) as f:
        for r in csv.DictReader(f):
            if not rx.search(r["Kernel_Name"]):
                continue
            name = r["Kernel_Name"]
            d = r.get("Dispatch_Id") or r.get("Correlation_Id")
            per.setdefault(r["Counter_Name"], {})[d] = float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                durs[d] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    if not per:
        raise SystemExit(f"no rows for /{regex}/ in {path}")
    vals = {c: list(v.values()) for c, v in per.items()}
    return vals, list(durs.values()), name


def summarize(a) -> None:
    vals, durs, name = read(a.csv, a.kernel_regex)
    med = {c: statistics.median(v) for c, v in vals.items()}
    n = max(len(v) for v in vals.values())
    lines = [f"# MFMA counters: {a.title}", "", f"kernel: {name}"]
    if a.source:
        lines.append(f"kernel sources (code without comments) sha256[:16]: "
                     f"{TR.source_hash(a.source)}  "
                     f"({', '.join(os.path.basename(p) for p in a.source)})")
    lines += ["command (from the repository root, one pass, all counters in one run):",
              f"  {a.command}", "", f"dispatches: {n} (medians below)"]
    dur = statistics.median(durs) * 1e-9 if durs else None
    if dur:
        lines.append(f"duration per dispatch (counter run): {dur * 1e3:.4f} ms")
    for c in COUNTERS:
        if c in med:
            lines.append(f"  {c:<32} {med[c]:.6g}")
    lines += ["", "derived (rocprofv3's MfmaUtil / MfmaFlopsBF16 definitions; GRBM_GUI_ACTIVE "
              f"is summed over the {XCDS} XCDs):"]
    cyc = med.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    if cyc:
        lines.append(f"  busy shader-clock cycles per XCD      GRBM_GUI_ACTIVE/{XCDS}"
                     f"             = {cyc:.4g}")
        if dur:
            lines.append(f"  effective shader clock                 cycles / duration"
                         f"             = {cyc / dur / 1e9:.3f} GHz (nominal 2.4)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            util = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
            lines.append(f"  MFMA utilisation                       MFMA_BUSY / (cycles x "
                         f"{SIMDS})   = {100 * util:.1f}%")
            if dur:
                lines.append(f"  MFMA busy vs 2.4 GHz x duration"
                             f"                                      = "
                             f"{100 * med['SQ_VALU_MFMA_BUSY_CYCLES'] / (2.4e9 * dur * SIMDS):.1f}%")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        ex = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        lines.append(f"  bf16 MFMA flops executed               MOPS_BF16 x 512"
                     f"               = {ex:.4g}")
        if dur:
            lines.append(f"  executed bf16 TFLOP/s in the counter run"
                         f"                             = {ex / dur / 1e12:.1f}")
        if a.alg_flops:
            lines.append(f"  algorithmic flops per dispatch ({a.alg_flops_label})"
                         f" = {a.alg_flops:.4g}")
            lines.append(f"  executed / algorithmic (row padding of the 256-row tiles)"
                         f"            = {ex / a.alg_flops:.4f}")
            if dur:
                lines.append(f"  algorithmic TFLOP/s in the counter run"
                             f"                               = {a.alg_flops / dur / 1e12:.1f} "
                             f"({100 * a.alg_flops / dur / PEAK_BF16:.1f}% of 2.5 PFLOP/s)")
    if "SQ_WAVE_CYCLES" in med:
        wc = med["SQ_WAVE_CYCLES"]
        if "SQ_WAIT_ANY" in med:
            lines.append(f"  share of wave time waiting on anything SQ_WAIT_ANY / SQ_WAVE_CYCLES"
                         f"  = {100 * med['SQ_WAIT_ANY'] / wc:.1f}%")
        if "SQ_WAIT_INST_ANY" in med:
            lines.append(f"  share of wave time with no issue       SQ_WAIT_INST_ANY / "
                         f"WAVE_CYCLES = {100 * med['SQ_WAIT_INST_ANY'] / wc:.1f}%")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("out")
    s.add_argument("--csv", required=True)
    s.add_argument("--kernel-regex", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--alg-flops", type=float, default=None)
    s.add_argument("--alg-flops-label", default="given")
    s.add_argument("--source", action="append", default=[])
    a = ap.parse_args(argv)
    summarize(a)


if __name__ == "__main__":
    main()
