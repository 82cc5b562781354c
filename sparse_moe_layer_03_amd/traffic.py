"""HBM traffic of a kernel from rocprofv3 counters, calibrated on a copy.

    python -m sparse_moe_layer_03_amd.traffic probe
        Runs a plain device-to-device copy of COPY_BYTES (3 times; torch's
        same-dtype copy_ is the runtime's copy kernel) so that FETCH_SIZE /
        WRITE_SIZE can be read for a transfer of known size.

    python -m sparse_moe_layer_03_amd.traffic summarize OUT.txt \\
        --kernel-fetch K.csv --kernel-write K.csv --copy-fetch C.csv \\
        --copy-write C.csv --kernel-regex REGEX --copy-regex REGEX \\
        --source FILE [--source FILE ...] --command "..."
        Reads rocprofv3 counter_collection CSVs (one counter per run) and
        writes a text summary: per-dispatch KiB of the kernel, the copy's
        KiB per KiB actually moved (the scale), the kernel's scaled bytes per
        launch, and a hash of the kernel's sources without comments (a
        reader of the summary can tell whether the kernel's code changed
        since the counters were taken).  When the regex matches several
        kernels (one call of the operation launches each once), the figures
        are per call: the sum over those kernels of their per-dispatch
        medians.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics
import sys

COPY_BYTES = 1 << 30


def code_text(text: str) -> str:
    """The code of a C++/HIP source: // comments and blank lines removed, so
    that editing a comment does not invalidate measured counters."""
    out = []
    for line in text.splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line.strip():
            out.append(line)
    return "\n".join(out)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in sorted(paths):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def probe() -> None:
    import torch

    n = COPY_BYTES // 2
    src = torch.full((n,), 1.0, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3", flush=True)


def per_kernel(path, regex, counter):
    """{kernel name: [counter value per dispatch]} for the kernels matching regex."""
    vals = {}
    rx = re.compile(regex)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and rx.search(r["Kernel_Name"]):
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for /{regex}/ in {path}")
    return vals


def per_dispatch(path, regex, counter):
    return [v for vs in per_kernel(path, regex, counter).values() for v in vs]


def summarize(a) -> None:
    kf = per_kernel(a.kernel_fetch, a.kernel_regex, "FETCH_SIZE")
    kw = per_kernel(a.kernel_write, a.kernel_regex, "WRITE_SIZE")
    cf = per_dispatch(a.copy_fetch, a.copy_regex, "FETCH_SIZE")
    cw = per_dispatch(a.copy_write, a.copy_regex, "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    s_f = statistics.median(cf) / kib    # counter KiB per KiB really read
    s_w = statistics.median(cw) / kib
    f_kib = sum(statistics.median(v) for v in kf.values())   # per call
    w_kib = sum(statistics.median(v) for v in kw.values())
    fetch_b = f_kib * 1024.0 / s_f
    write_b = w_kib * 1024.0 / s_w
    lines = [
        f"# HBM traffic per launch of /{a.kernel_regex}/ (rocprofv3 --pmc, one counter per run)",
        f"# command: {a.command}",
    ]
    if len(kf) > 1:
        lines.append(f"# {len(kf)} kernels per call; figures per call = sum of the per-kernel medians")
        for name in sorted(kf):
            lines.append(f"#   {name}: fetch {statistics.median(kf[name]):.1f} KiB, write "
                         f"{statistics.median(kw.get(name, [0.0])):.1f} KiB per dispatch "
                         f"(n={len(kf[name])})")
    nf = sum(len(v) for v in kf.values())
    nw = sum(len(v) for v in kw.values())
    lines += [
        f"kernel_fetch_kib_per_dispatch_median {f_kib:.1f}  (n={nf})",
        f"kernel_write_kib_per_dispatch_median {w_kib:.1f}  (n={nw})",
        f"copy_fetch_kib_per_dispatch_median {statistics.median(cf):.1f}  (copy of {COPY_BYTES} B)",
        f"copy_write_kib_per_dispatch_median {statistics.median(cw):.1f}",
        f"scale_fetch {s_f:.4f}  scale_write {s_w:.4f}  (counter KiB per KiB moved)",
        f"traffic_fetch_bytes {fetch_b:.0f}",
        f"traffic_write_bytes {write_b:.0f}",
        f"traffic_bytes {fetch_b + write_b:.0f}",
        f"source_hash {source_hash(a.source)}",
        "sources " + " ".join(os.path.relpath(p) for p in a.source),
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_summary(path):
    """Parse a summary written by summarize(); None if absent."""
    if not os.path.exists(path):
        return None
    out = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("#") or not ln.strip():
                continue
            k, v = ln.split(None, 1)
            out[k] = v.strip().split()[0] if k != "sources" else v.split()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("probe")
    s = sub.add_parser("summarize")
    s.add_argument("out")
    for k in ("kernel-fetch", "kernel-write", "copy-fetch", "copy-write", "kernel-regex",
              "copy-regex", "command"):
        s.add_argument("--" + k, required=True)
    s.add_argument("--source", action="append", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "probe":
        probe()
    else:
        summarize(a)


if __name__ == "__main__":
    sys.exit(main())
