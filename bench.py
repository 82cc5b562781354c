"""MoE layer forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: moe_route ->
moe_dispatch -> moe_ffn_gate_up -> moe_ffn_down -> moe_combine, plus
moe_pid_update on workloads that run the PID.  Inputs are resident in HBM
before timing starts.  Prints ONE JSON line.

Default (--workload headline): the prefill-shaped batch, T=16384 tokens,
d_model=6144, 512 SwiGLU experts (d_ff=2048) + 256 identity experts, top-12,
bf16, router bias 0 -- the line's `value`, `roofline` and `cpu_baseline` --
and, on the same resident weights (38.7 GB), the decode-shaped batch of
T=128 tokens, reported in the line's `decode` record with its own step time,
roofline and CPU baseline.  `metric_fracs` gives the two fractions the
metric is quoted in: prefill whole-layer MFMA fraction of the bf16 peak and
decode whole-layer HBM fraction.  --workload NAME runs one workload alone
(small_bf16 and skewed_bf16 run their PID over K batches: the timed steps are
batches 0..K-1, starting from the initial bias; warm-up steps are undone).

The steps are timed twice over the same batches and controller trajectory:
issued one call at a time with four HIP events each (step start, gate/up
start and end, down end: the step spread and the expert GEMM durations for
the roofline), and as one HIP graph per step, captured once and replayed (no
events inside).  `value` and `ms_per_step` come from the run named by
--launch (default: graph); both runs are reported, and the graph run's final
output and bias must equal the eager run's bit for bit.  After them, outside
the timed region, the same steps are replayed once with an event at every
stage boundary (stages_ms_mean) and every step's expert loads logged (exact
assignments and touched experts per step for the roofline, load variance per
batch), and, for the workloads whose data can stay in L2 / Infinity Cache,
once more with 512 MiB written between steps ("cold", event-timed steps
only).

`roofline` is the dominant kernel's (gate/up; `roofline_down` the down
GEMM's): algorithmic flops and bytes per launch over the event-measured
launch time, against whichever bound (bf16 MFMA 2.5 PFLOP/s, HBM 8 TB/s) the
algorithmic work reaches first.  `layer` is the whole step's, from each
step's exact FFN assignments A and touched FFN experts U: F = 2 T d E +
6 A d d_ff flops, B_min = the touched experts' weights, the router matrix, x,
y and the routing outputs; mfma_frac = sum F / (t * peak), hbm_frac = sum
B_min / (t * 8 TB/s), roofline_frac = sum max(F / peak, B_min / 8 TB/s) / t,
with t the wall time of the run that gives `value`.

`cpu_baseline` is the CPU oracle timed on the host cores after the GPU runs.
Small, skewed and tiny batches run whole; for the 512-expert model the
oracle routes, dispatches, gathers and combines every token, runs the expert
FFN of a seeded random subset of the touched experts on their rows, and the
FFN time is scaled by touched experts / subset size (the label says so).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense bf16 MFMA FLOP/s (MI355X)
PEAK_F32_MFMA = 157.3e12
PEAK_HBM = 8.0e12       # B/s
METRIC = "MoE-layer tokens/s at 1 GPU; % bf16 MFMA peak (prefill) / % HBM BW (decode)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "small_bf16", "decode_bf16", "prefill_bf16",
                             "skewed_bf16", "tiny_f32"],
                    help="headline (default) = prefill_bf16 with decode_bf16 on the same "
                         "weights in a sub-record")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph",
                    help="how the timed steps whose time gives `value` are launched: each "
                         "step captured once as a HIP graph and replayed (default; the eager "
                         "run is reported beside it), or the library calls issued one by one "
                         "(then no graph is captured, e.g. under a counter profiler)")
    ap.add_argument("--scmoe", type=int, default=0, metavar="D_FF",
                    help="shortcut-connected block: time the MoE layer against a dense "
                         "SwiGLU branch of this width on a second stream (e.g. 12288); "
                         "0 = off")
    ap.add_argument("--cu-split", default="",
                    help="with --scmoe: comma-separated CU counts for the dense branch; for "
                         "each, the MoE layer and the branch run on CU-masked streams with "
                         "disjoint CU sets (the layer gets the rest; contiguous CU ranges, the "
                         "masks the runtime accepts)")
    ap.add_argument("--eplb", default="",
                    help="SLOTS,DEVICES: after each batch's dispatch, plan the placement of "
                         "the FFN experts on SLOTS expert slots over DEVICES devices of an EP "
                         "domain (moe_eplb_plan) and report each batch's device max/mean load: "
                         "one expert per slot, the plan of the same batch, and the plan of the "
                         "previous batch applied to it")
    ap.add_argument("--layers", type=int, default=0,
                    help="chain this many resident layers (distinct weights, layer i's output "
                         "is layer i+1's input) and time the chain as one graph, against the "
                         "same layers timed one at a time; with --prefetch, the next layer's "
                         "router matrix is read on a second stream while a layer's expert "
                         "GEMMs run (Infinity Cache warm-up)")
    ap.add_argument("--prefetch", action="store_true")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the named workload's model and value distributions at this many "
                         "tokens per batch instead (a batch-size sweep; the config is named "
                         "<workload>@T<tokens>); not for the default headline run")
    ap.add_argument("--balance", type=float, default=0.0,
                    help="per-expert load-balancing step (moe_balance_update) after the PID; "
                         "0 = off")
    return ap.parse_args()


def gate_up_units(w, A, U):
    """Algorithmic work of one moe_ffn_gate_up launch.
    flops: 2 GEMMs of A x d_model x d_ff.  bytes: gate+up weights of the U
    touched experts, the A gathered token rows, and H written once."""
    el = 2 if w.dtype == "bf16" else 4
    flops = 4.0 * A * w.d_model * w.d_ff
    byts = el * (2.0 * U * w.d_ff * w.d_model + A * w.d_model + A * w.d_ff)
    return flops, byts


def down_kernel_name(w):
    """The down GEMM's kernel for this shape."""
    name = gate_up_kernel_name(w)
    if name.startswith("grouped_gemm_big_kernel"):
        return ("grouped_gemm_big_kernel<2,4,1|2> (320x192 tiles for the experts of 257..320 "
                "rows when they fill 4 rounds of the grid, then 256x256 tiles on 16x16x32 MFMAs "
                "for the rest; down; event time of both launches)")
    return (name.replace("gate/up + SwiGLU", "down").replace("mode 1", "mode 2")
            .replace("16x256", "16x128"))


def gate_up_kernel_name(w):
    """Which gate/up kernel the library launches for this shape (the same
    tests the library makes: at least 32 assignments per expert and at least
    64 tiles, or at least 64 assignments per FFN expert, for the tall tiles;
    bf16 and both K lengths multiples of 128 for the 256x256 direct-to-LDS
    tiles)."""
    E = w.n_ffn + w.n_zero
    Tk = w.T * w.top_k
    cdiv = lambda a, b: -(-a // b)  # noqa: E731
    tall = ((Tk // E >= 32 and cdiv(Tk, 128) * cdiv(min(w.d_ff, w.d_model), 128) >= 64)
            or Tk // w.n_ffn >= 64)
    if (tall and w.dtype == "bf16" and w.d_model % 128 == 0 and w.d_ff % 128 == 0
            and cdiv(Tk, 256) * min(w.d_ff // 128, w.d_model // 256) >= 64):
        if w.d_model >= 4096:  # the 256x256 tiles on 16x16x32 MFMAs from d_model 4096
            return ("grouped_gemm_big_kernel<1,4,1|2> (320x192 tiles for the experts of "
                    "257..320 rows when they fill 4 rounds of the grid, then 256x256 tiles on "
                    "16x16x32 MFMAs for the rest; gate/up + SwiGLU; event time of both launches)")
        return ("grouped_gemm_big_kernel<1,4,1|0> (320x192 tiles for the experts of 257..320 "
                "rows when they fill 4 rounds of the grid, then 256x256 tiles for the rest; "
                "gate/up + SwiGLU; event time of both launches)")
    if tall:
        return "grouped_gemm_kernel mode 1 (128x128 tiles, gate/up + SwiGLU)"
    return "grouped_gemm_kernel mode 1 (16x256 tiles, gate/up + SwiGLU)"


def measured_traffic(workload, kernel="gate_up"):
    """HBM bytes per gate/up (or down) launch from the committed counter
    summary of this workload, or None when there is none or the GEMM
    sources changed since the counters were taken."""
    from sparse_moe_layer_03_amd import traffic as TR

    summ = TR.read_summary(os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt"))
    if not summ:
        return None
    srcs = [os.path.join(ROOT, p) for p in summ.get("sources", [])]
    if not srcs or not all(os.path.exists(p) for p in srcs):
        return None
    if TR.source_hash(srcs) != summ.get("source_hash"):
        return None
    return float(summ["traffic_bytes"])


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, m, budget_s=12.0):
    """Time the oracle (as it stands) on the host cores: whole batches of the
    workload, in order, until about ``budget_s`` seconds of oracle work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O
    from sparse_moe_layer_03_amd import synth as S

    wr = S.to_numpy64(m["wr"])
    lb = None if m["lb"] is None else m["lb"].cpu().numpy().astype(np.float64)
    bias = m["bias0"].cpu().numpy().astype(np.float64)
    wg, wu, wd = S.to_numpy64(m["wg"]), S.to_numpy64(m["wu"]), S.to_numpy64(m["wd"])
    st = O.PidState()
    t_total, n_tok, nb = 0.0, 0, 0
    while t_total < budget_s and nb < len(m["xs"]):
        x = S.to_numpy64(m["xs"][nb])
        t0 = time.perf_counter()
        out = O.forward(x, wr, bias.astype(np.float32), wg, wu, wd, w.n_ffn, w.top_k,
                        w.routed_scaling, lb)
        if w.pid:
            bias, st, _ = O.pid_update(out["counts"], w.n_ffn, x.shape[0], bias, st, *w.pid)
        t_total += time.perf_counter() - t0
        n_tok += x.shape[0]
        nb += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return n_tok / t_total, threads, t_total, nb


def cpu_baseline_sampled(w, m, x, budget_s=12.0, min_experts=4, seed=0):
    """Time the oracle (as it stands) on one batch of the 512-expert model.

    Every token is routed, dispatched, gathered and combined by the oracle;
    the expert FFN runs on a seeded random subset of the touched experts
    (on all their rows) until about ``budget_s`` seconds of FFN work, and its
    time is scaled by (touched experts / subset size).  bf16 -> float64
    conversion of inputs and weights is left out of the timed work.
    Returns (tokens/s, threads, label)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O
    from sparse_moe_layer_03_amd import synth as S

    wr = S.to_numpy64(m["wr"])
    lb = None if m["lb"] is None else m["lb"].cpu().numpy().astype(np.float64)
    bias = m["bias0"].cpu().numpy().astype(np.float32)
    x64 = S.to_numpy64(x)
    t0 = time.perf_counter()
    r = O.route(x64, wr, bias, w.top_k, w.routed_scaling, lb)
    d = O.dispatch(r["topk_idx"], w.E)
    n_rows = int(d["offsets"][w.n_ffn])
    xp = O.gather_rows(x64, d["perm"], w.top_k, n_rows)
    t_front = time.perf_counter() - t0
    counts = d["counts"][: w.n_ffn]
    touched = np.nonzero(counts)[0]
    order = np.random.default_rng(seed).permutation(touched)
    y_perm = np.zeros((n_rows, w.d_model))
    t_ffn, done, rows = 0.0, 0, 0
    wall0 = time.perf_counter()
    for e in order:
        lo, hi = int(d["offsets"][e]), int(d["offsets"][e + 1])
        wg, wu, wd = (S.to_numpy64(m["wg"][e]), S.to_numpy64(m["wu"][e]),
                      S.to_numpy64(m["wd"][e]))
        t1 = time.perf_counter()
        y_perm[lo:hi] = O.swiglu_ffn(xp[lo:hi], wg, wu, wd)
        t_ffn += time.perf_counter() - t1
        done += 1
        rows += hi - lo
        # stop on FFN time, or on wall time (the untimed weight conversion
        # dominates when experts hold few rows)
        if done >= min_experts and (t_ffn >= budget_s
                                    or time.perf_counter() - wall0 >= 2.5 * budget_s):
            break
    t2 = time.perf_counter()
    O.combine(x64, y_perm, r["topk_idx"], r["topk_gate"], d["inv_perm"], w.n_ffn)
    t_comb = time.perf_counter() - t2
    scale = len(touched) / done
    total = t_front + t_ffn * scale + t_comb
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    label = (f"one batch of {w.T} tokens: oracle route+dispatch+gather {t_front:.2f} s and "
             f"combine {t_comb:.2f} s over all tokens; expert FFN on {done} of the "
             f"{len(touched)} touched experts ({rows} of {n_rows} rows, seeded random subset) "
             f"{t_ffn:.2f} s, scaled x{scale:.1f}; float64")
    return w.T / total, threads, label


def scmoe_main(args):
    """MoE layer and the dense SwiGLU branch of a shortcut-connected block:
    each alone, one after the other on one stream, and concurrently on two
    streams (default priorities).  One step = the layer and the branch over
    one batch; value = tokens/s of the concurrent steps."""
    import numpy as np
    import torch

    from sparse_moe_layer_03_amd import binding as B
    from sparse_moe_layer_03_amd import scmoe
    from sparse_moe_layer_03_amd import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    w = S.WORKLOADS[args.workload]
    if w.pid or w.zipf_s:
        print("--scmoe runs the decode/prefill workloads (fixed router bias)", file=sys.stderr)
        sys.exit(2)
    wr = S.make_router(w, dev)
    bias = S.make_bias(w, dev)
    wg, wu, wd = S.make_experts(w, dev)
    x = S.make_x(w, 0, dev)
    w1, w3, w2 = S.make_dense(w, args.scmoe, dev)
    shape = B.make_shape(w.T, w.d_model, w.n_ffn, w.n_zero, w.d_ff, w.top_k, w.dtype,
                         w.routed_scaling)
    buf = B.LayerBuffers(shape, dev)
    br = scmoe.DenseBranch(w.T, w.d_model, args.scmoe, w.dtype, dev)
    main_s = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def moe():
        B.layer_forward(buf, x, wr, bias, wg, wu, wd)

    def dense(stream=None):
        br.run(x, w1, w3, w2, stream=stream)

    def both_serial():
        moe()
        dense()

    def both_concurrent():
        side.wait_stream(main_s)
        moe()
        with torch.cuda.stream(side):
            dense(side)
        main_s.wait_stream(side)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    # CU-partitioned variants: the layer and the branch on CU-masked streams
    # with disjoint CU sets (default priority)
    masked = {}
    n_cus = B.moe_device_cu_count()
    for part in [int(v) for v in args.cu_split.split(",") if v.strip()]:
        for pattern in ("contiguous",):
            d_words = scmoe.cu_mask(n_cus, 0, part, pattern)
            m_words = [(~v) & 0xFFFFFFFF for v in d_words]
            if n_cus % 32:
                m_words[-1] &= (1 << (n_cus % 32)) - 1
            masked[f"{pattern}_dense{part}"] = (scmoe.MaskedStream(m_words),
                                                scmoe.MaskedStream(d_words))

    def masked_concurrent(key):
        ms_, ds_ = masked[key]

        def fn():
            ms_.stream.wait_stream(main_s)
            ds_.stream.wait_stream(main_s)
            with torch.cuda.stream(ms_.stream):
                B.layer_forward(buf, x, wr, bias, wg, wu, wd, stream=ms_.stream)
            with torch.cuda.stream(ds_.stream):
                br.run(x, w1, w3, w2, stream=ds_.stream)
            main_s.wait_stream(ms_.stream)
            main_s.wait_stream(ds_.stream)
        return fn

    # interleave the modes over three rounds; keep each mode's best round
    res = {k: [] for k in ["moe", "dense", "serial", "concurrent"] + list(masked)}
    for _ in range(3):
        res["moe"].append(timed(moe))
        res["dense"].append(timed(dense))
        res["serial"].append(timed(both_serial))
        res["concurrent"].append(timed(both_concurrent))
        for key in masked:
            res[key].append(timed(masked_concurrent(key)))
    for ms_, ds_ in masked.values():
        ms_.close()
        ds_.close()
    ms = {k: float(np.min(v)) for k, v in res.items()}
    dense_flops = 6.0 * w.T * w.d_model * args.scmoe
    line = {
        "metric": METRIC + " (shortcut-connected block: MoE layer || dense FFN branch)",
        "value": w.T / (ms["concurrent"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms["concurrent"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/d_in) weights)",
        "config": {"workload": f"{w.name}+dense{args.scmoe}", "T": w.T, "d_model": w.d_model,
                   "n_ffn": w.n_ffn, "n_zero": w.n_zero, "d_ff": w.d_ff, "top_k": w.top_k,
                   "dense_d_ff": args.scmoe},
        "scmoe": {"moe_ms": ms["moe"], "dense_ms": ms["dense"], "serial_ms": ms["serial"],
                  "concurrent_ms": ms["concurrent"],
                  "saved_ms": ms["serial"] - ms["concurrent"],
                  "dense_hidden_frac": (ms["serial"] - ms["concurrent"]) / ms["dense"],
                  "dense_weight_gb_per_s": 3.0 * w.d_model * args.scmoe
                  * (2 if w.dtype == "bf16" else 4) / (ms["dense"] * 1e-3) / 1e9,
                  "dense_tflop_per_s": dense_flops / (ms["dense"] * 1e-3) / 1e12,
                  "cu_partitioned_ms": {k: ms[k] for k in masked},
                  "rounds_ms": res},
    }
    print(json.dumps(line), flush=True)


def eplb_report(w, loads, eplb, dispatch_ms):
    """Per-batch device max/mean FFN load of the expert placement plans
    (counts of each batch from the load log): experts one per slot in id
    order (expert e on device e * D // N), the plan made from the same
    batch, and the plan of the previous batch applied to this batch's
    counts (each expert's rows split over its replicas as the plan does)."""
    import numpy as np

    D = eplb["D"]
    rep = eplb["rep"].cpu().numpy()
    sdev = eplb["sdev"].cpu().numpy()
    dload = eplb["dload"].cpu().numpy().astype(np.int64)
    N = w.n_ffn

    def ratio(v):
        v = np.asarray(v, np.float64)
        return round(float(v.max() / max(v.mean(), 1e-12)), 3)

    def apply(counts, r, devs):
        out = np.zeros(D, np.int64)
        s = 0
        for e in range(N):
            c = int(counts[e])
            for j in range(int(r[e])):
                out[devs[s]] += (j + 1) * c // int(r[e]) - j * c // int(r[e])
                s += 1
        return out

    K = loads.shape[0]
    naive = [ratio(np.bincount(np.arange(N) * D // N, weights=loads[i, :N], minlength=D))
             for i in range(K)]
    same = [ratio(dload[i]) for i in range(K)]
    prev = [None] + [ratio(apply(loads[i, :N], rep[i - 1], sdev[i - 1])) for i in range(1, K)]
    return {"slots": eplb["S"], "devices": D,
            "device_max_over_mean_one_expert_per_slot": naive,
            "device_max_over_mean_planned_same_batch": same,
            "device_max_over_mean_planned_previous_batch": prev,
            "dispatch_plus_plan_ms_mean": float(np.mean(dispatch_ms)),
            "replicas_of_the_hottest_expert_last_batch": int(rep[K - 1].max())}


def build_model(w, dev):
    """Resident synthetic weights and router state of a workload."""
    from sparse_moe_layer_03_amd import synth as S

    alpha = None
    if w.zipf_s:
        with open(os.path.join(ROOT, "tests", "golden", "zipf_alpha.json")) as f:
            alpha = json.load(f)["alpha"]
    wg, wu, wd = S.make_experts(w, dev)
    return dict(wr=S.make_router(w, dev), bias0=S.make_bias(w, dev),
                lb=S.zipf_logit_offset(w, alpha, dev) if w.zipf_s else None,
                wg=wg, wu=wu, wd=wd)


def kernel_roofline(name, fl, by, secs, peak_fl):
    """Roofline of one kernel from its algorithmic flops and bytes per
    launch and its measured launch times (seconds)."""
    import numpy as np

    t_fl = np.sum(fl) / peak_fl
    t_by = np.sum(by) / PEAK_HBM
    tot = float(np.sum(secs))
    if t_fl >= t_by:
        roof = {"bound": "mfma", "achieved": float(np.sum(fl) / tot / 1e12),
                "peak": peak_fl / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": float(np.sum(by) / tot / 1e9),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # both fractions, whichever bound applies
    roof["mfma_frac"] = float(np.sum(fl) / tot / peak_fl)
    roof["hbm_frac"] = float(np.sum(by) / tot / PEAK_HBM)
    roof["kernel"] = "%s, mean %.4f ms/launch" % (name, tot / len(secs) * 1e3)
    return roof


def run_workload(w, args, mdl, dev, cpu=True):
    """Time K steps of workload ``w`` on resident weights ``mdl``; returns
    the JSON record."""
    import numpy as np
    import torch

    from sparse_moe_layer_03_amd import binding as B
    from sparse_moe_layer_03_amd import synth as S

    wr, bias0, lb = mdl["wr"], mdl["bias0"], mdl["lb"]
    wg, wu, wd = mdl["wg"], mdl["wu"], mdl["wd"]
    bias = bias0.clone()
    n_x = min(max(args.steps, 1), w.batches) if w.pid else 1
    xs = [S.make_x(w, b, dev) for b in range(n_x)]
    shape = B.make_shape(w.T, w.d_model, w.n_ffn, w.n_zero, w.d_ff, w.top_k, w.dtype,
                         w.routed_scaling)
    buf = B.LayerBuffers(shape, dev)
    params = B.MoePidParams(*w.pid) if w.pid else None
    r_log = torch.zeros(max(args.steps, 1) + args.warmup + 1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    load_log = None
    eplb = None
    if args.eplb:
        n_slots, n_dev = (int(v) for v in args.eplb.split(","))
        i32 = dict(dtype=torch.int32, device=dev)
        Kp = max(args.steps, 1)
        eplb = dict(S=n_slots, D=n_dev, rep=torch.zeros((Kp, w.n_ffn), **i32),
                    sexp=torch.zeros((Kp, n_slots), **i32),
                    srows=torch.zeros((Kp, n_slots, 2), **i32),
                    sdev=torch.zeros((Kp, n_slots), **i32),
                    dload=torch.zeros((Kp, n_dev), **i32))

    def step(i, ev=None):
        """One step; ev: None, 7 events (every stage boundary) or 4 events
        (step start, gate/up start, gate/up end, down end: the timed run
        keeps its event count low, since each record costs GPU time)."""
        x = xs[i % len(xs)]
        full = ev is not None and len(ev) == 7
        if ev is not None:
            ev[0].record(stream)
        B.moe_route(shape, x, wr, lb, bias, buf.topk_idx, buf.topk_gate, None, buf.ws)
        if full:
            ev[1].record(stream)
        B.moe_dispatch(shape, buf.topk_idx, x, buf.counts, buf.offsets, buf.perm,
                       buf.inv_perm, None, buf.ws)
        if eplb is not None:
            j = i % eplb["rep"].shape[0]
            B.moe_eplb_plan(shape, eplb["S"], eplb["D"], buf.counts, buf.offsets,
                            eplb["rep"][j], eplb["sexp"][j], eplb["srows"][j], eplb["sdev"][j],
                            eplb["dload"][j])
        if ev is not None:
            ev[2 if full else 1].record(stream)
        B.moe_ffn_gate_up(shape, x, None, buf.perm, buf.offsets, wg, wu, buf.ws)
        if ev is not None:
            ev[3 if full else 2].record(stream)
        B.moe_ffn_down(shape, buf.offsets, wd, buf.y_perm, buf.ws)
        if ev is not None:
            ev[4 if full else 3].record(stream)
        B.moe_combine(shape, x, buf.y_perm, buf.topk_idx, buf.topk_gate, buf.inv_perm, buf.y)
        if full:
            ev[5].record(stream)
        if params is not None:
            B.moe_pid_update(shape, params, buf.counts, buf.pid_state, bias, r_log,
                             r_log.numel())
        if args.balance > 0:
            B.moe_balance_update(shape, args.balance, buf.counts, bias)
        if load_log is not None:
            load_log[i % load_log.shape[0]].copy_(buf.counts)
        if full:
            ev[6].record(stream)

    def reset_controller():
        bias.copy_(bias0)
        buf.pid_state.zero_()
        r_log.zero_()
        torch.cuda.synchronize()

    # ---- warm-up, then restore the initial controller state
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    reset_controller()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    ev_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, evs[i])
    ev_end.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # ---- timed-run durations (HIP events on the launch stream): each step
    # (start to next start), each gate/up and each down launch
    starts = [evs[i][0] for i in range(K)] + [ev_end]
    step_ms = np.array([starts[i].elapsed_time(starts[i + 1]) for i in range(K)])
    gu_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in range(K)])
    dn_ms = np.array([evs[i][2].elapsed_time(evs[i][3]) for i in range(K)])

    # ---- the same K steps as HIP graphs: each step (its batch differs) is
    # captured once, the controller is reset, all graphs are replayed once
    # untimed and once timed.  Same kernels, same launches, same inputs and
    # controller trajectory: the final output and bias must equal the eager
    # run's bit for bit.
    y_eager, bias_eager = buf.y.clone(), bias.clone()
    g_elapsed, graph_match = None, None
    graphs = [] if args.launch == "graph" else None
    cap = torch.cuda.Stream()  # default priority
    for i in range(K if graphs is not None else 0):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            step(i)
        graphs.append(gr)
    if graphs is not None:
        for _ in range(2):
            reset_controller()
            g0 = time.perf_counter()
            for gr in graphs:
                gr.replay()
            torch.cuda.synchronize()
            g_elapsed = time.perf_counter() - g0
        graph_match = bool(torch.equal(buf.y, y_eager) and torch.equal(bias, bias_eager))
        if not graph_match:
            print("bench.py: graph replay differs from the eager run", file=sys.stderr)
            sys.exit(1)
        del graphs
    eager_elapsed = elapsed
    if args.launch == "graph":
        elapsed = g_elapsed

    # ---- untimed replay of the same K steps (same inputs, same controller
    # trajectory) with an event at every stage boundary and each step's
    # expert loads logged: the stage breakdown and exact per-step A and U
    reset_controller()
    load_log = torch.zeros((K, w.n_ffn + w.n_zero), dtype=torch.int32, device=dev)
    revs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    for i in range(K):
        step(i, revs[i])
    torch.cuda.synchronize()
    names = ["route", "dispatch", "ffn_gate_up", "ffn_down", "combine", "pid"]
    st_ms = {n: [revs[i][j].elapsed_time(revs[i][j + 1]) for i in range(K)]
             for j, n in enumerate(names)}
    loads = load_log.cpu().numpy().astype(np.int64)
    load_log = None
    A = loads[:, : w.n_ffn].sum(axis=1)
    U = (loads[:, : w.n_ffn] > 0).sum(axis=1)

    # ---- cold pass: 512 MiB written between steps evicts L2 and the
    # Infinity Cache, so every step starts from HBM (events time the step
    # only); for the workloads whose data can stay cache-resident
    cold = None
    if w.name in ("tiny_f32", "small_bf16", "skewed_bf16"):
        reset_controller()
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
        for i in range(K):
            scratch.fill_(i & 255)
            step(i, cevs[i])
        torch.cuda.synchronize()
        del scratch
        c_ms = np.array([cevs[i][0].elapsed_time(cevs[i][6]) for i in range(K)])
        cold = {"ms_per_step_median": float(np.median(c_ms)),
                "tokens_per_s_median": w.T / (float(np.median(c_ms)) * 1e-3),
                "ffn_gate_up_ms_mean": float(np.mean(
                    [cevs[i][2].elapsed_time(cevs[i][3]) for i in range(K)]))}
    reset_controller()

    el = 2 if w.dtype == "bf16" else 4
    peak_fl = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32_MFMA
    fl, by = zip(*[gate_up_units(w, int(a), int(u)) for a, u in zip(A, U)])
    roof = kernel_roofline(gate_up_kernel_name(w), fl, by, gu_ms / 1e3, peak_fl)
    roof["traffic"] = measured_traffic(w.name)
    # down: 2 A d d_ff flops; the U experts' down weights, H rows in, y_perm rows out
    fl_d = [2.0 * a * w.d_model * w.d_ff for a in A]
    by_d = [el * (1.0 * u * w.d_model * w.d_ff + a * w.d_ff + a * w.d_model)
            for a, u in zip(A, U)]
    roof_d = kernel_roofline(down_kernel_name(w), fl_d, by_d, dn_ms / 1e3, peak_fl)
    roof_d["traffic"] = measured_traffic(w.name, "down")

    # whole-layer figures per step from its exact A (FFN assignments) and U
    # (touched FFN experts): F = 2 T d E + 6 A d d_ff flops; B_min = the
    # touched experts' weights + router matrix + x and y + idx and gates
    E_ = w.n_ffn + w.n_zero
    F = 2.0 * w.T * w.d_model * E_ + 6.0 * A * w.d_model * w.d_ff
    Bmin = (3.0 * el * U * w.d_model * w.d_ff + el * E_ * w.d_model + 2.0 * el * w.T * w.d_model
            + 8.0 * w.T * w.top_k)
    tstar = np.maximum(F / peak_fl, Bmin / PEAK_HBM)
    layer = {"flop_per_step": float(F.mean()), "bytes_min_per_step": float(Bmin.mean()),
             "mfma_frac": float(F.sum() / (elapsed * peak_fl)),
             "hbm_frac": float(Bmin.sum() / (elapsed * PEAK_HBM)),
             "roofline_frac": float(tstar.sum() / elapsed),
             "bound": "mfma" if (F / peak_fl).sum() >= (Bmin / PEAK_HBM).sum() else "hbm"}

    value = w.T * K / elapsed
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/d_in) weights)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d_model, "n_ffn": w.n_ffn,
                   "n_zero": w.n_zero, "d_ff": w.d_ff, "top_k": w.top_k,
                   "pid": list(w.pid) if w.pid else None},
        "roofline": roof,
        "roofline_down": roof_d,
        "layer": layer,
        "step_ms": {"median": float(np.median(step_ms)), "p10": float(np.percentile(step_ms, 10)),
                    "p90": float(np.percentile(step_ms, 90))},
        "stages_ms_mean": {n: float(np.mean(v)) for n, v in st_ms.items()},
        "launch": args.launch,
        "graph": None if g_elapsed is None else {
            "tokens_per_s": w.T * K / g_elapsed, "ms_per_step": g_elapsed / K * 1e3,
            "matches_eager": graph_match},
        "eager": {"tokens_per_s": w.T * K / eager_elapsed,
                  "ms_per_step": eager_elapsed / K * 1e3},
        "ffn_assignments_per_step_mean": float(np.mean(A)),
        "touched_ffn_experts_per_step_mean": float(np.mean(U)),
    }
    if cold is not None:
        line["cold"] = cold
    if w.pid:
        line["r_per_step"] = [round(float(a) / w.T, 4) for a in A]
        line["ms_per_batch"] = [round(float(v), 4) for v in step_ms]
        # each batch's whole-layer roofline fraction: max(F/peak, B_min/HBM)
        # over its event-timed (eager) step time
        line["layer_roofline_frac_per_batch"] = [
            round(float(ts / (ms * 1e-3)), 3) for ts, ms in zip(tstar, step_ms)]
        ll = loads[:, : w.n_ffn].astype(np.float64)
        line["ffn_load_max_over_mean_per_step"] = [
            round(float(r.max() / max(r.mean(), 1e-9)), 2) for r in ll]
        line["ffn_load_variance_per_step"] = [round(float(r.var()), 1) for r in ll]
    if args.balance > 0:
        line["balance_gamma"] = args.balance
    if eplb is not None:
        line["eplb"] = eplb_report(w, loads, eplb, st_ms["dispatch"])

    line["cpu_baseline"] = None
    if cpu and not args.no_cpu_baseline:
        if w.name in ("small_bf16", "skewed_bf16", "tiny_f32"):
            m = dict(mdl, xs=xs)
            v, threads, secs, nb = cpu_baseline(w, m)
            sample = (f"first {nb} whole batch(es) ({nb * w.T} tokens) of the same workload "
                      f"and inputs: oracle route+dispatch+FFN+combine"
                      f"{'+PID' if w.pid else ''} in float64, {secs:.1f} s")
        else:
            v, threads, sample = cpu_baseline_sampled(w, mdl, xs[0])
        line["cpu_baseline"] = {"value": v, "unit": "tokens/s", "cores": threads,
                                "kind": "oracle", "cpu": cpu_model(),
                                "host_cpus": os.cpu_count(), "sample": sample}
    return line


def chain_main(args):
    """Several resident MoE layers back to back (decode or prefill shape):
    each layer's output is the next layer's input.  Times (a) every layer
    alone, each captured as its own graph, and (b) the chain captured as
    one graph, optionally with the next layer's router matrix read into the
    cache hierarchy on a side stream while the current layer's expert GEMMs
    run.  value = tokens/s of the chain (one step = all layers)."""
    import dataclasses

    import numpy as np
    import torch

    from sparse_moe_layer_03_amd import binding as B
    from sparse_moe_layer_03_amd import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    base = S.WORKLOADS[args.workload]
    L = args.layers
    ws = [dataclasses.replace(base, seed=base.seed + 101 * i) for i in range(L)]
    print(f"bench.py: {L} layers of {base.name}, "
          f"{L * base.expert_weight_bytes() / 1e9:.0f} GB of expert weights", file=sys.stderr,
          flush=True)
    mdls = [build_model(w, dev) for w in ws]
    shape = B.make_shape(base.T, base.d_model, base.n_ffn, base.n_zero, base.d_ff, base.top_k,
                         base.dtype, base.routed_scaling)
    bufs = [B.LayerBuffers(shape, dev) for _ in range(L)]
    x0 = S.make_x(base, 0, dev)
    side = torch.cuda.Stream()  # default priority
    sink = torch.empty_like(mdls[0]["wr"])
    evs = [torch.cuda.Event() for _ in range(L)]

    def layer(i, x, prefetch):
        m, buf = mdls[i], bufs[i]
        B.moe_route(shape, x, m["wr"], m["lb"], m["bias0"], buf.topk_idx, buf.topk_gate, None,
                    buf.ws)
        B.moe_dispatch(shape, buf.topk_idx, x, buf.counts, buf.offsets, buf.perm, buf.inv_perm,
                       None, buf.ws)
        cur = torch.cuda.current_stream()
        if prefetch and i + 1 < L:
            evs[i].record(cur)
            side.wait_event(evs[i])
            with torch.cuda.stream(side):
                # read the next router matrix (a plain copy: no reduction, no
                # memset in the graph) while this layer's GEMMs stream weights
                sink.copy_(mdls[i + 1]["wr"])
        B.moe_ffn_gate_up(shape, x, None, buf.perm, buf.offsets, m["wg"], m["wu"], buf.ws)
        B.moe_ffn_down(shape, buf.offsets, m["wd"], buf.y_perm, buf.ws)
        B.moe_combine(shape, x, buf.y_perm, buf.topk_idx, buf.topk_gate, buf.inv_perm, buf.y)
        if prefetch and i + 1 < L:
            cur.wait_stream(side)
        return buf.y

    def chain(prefetch):
        x = x0
        for i in range(L):
            x = layer(i, x, prefetch)
        return x

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            fn()
        return g

    def timed(g, reps):
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    # reference outputs (eager chain) for the bitwise check of every variant
    y_ref = chain(False).clone()
    torch.cuda.synchronize()
    singles = [capture(lambda i=i: layer(i, x0 if i == 0 else bufs[i - 1].y, False))
               for i in range(L)]
    g_chain = capture(lambda: chain(False))
    g_pref = capture(lambda: chain(True)) if args.prefetch else None
    res = {"layers_one_at_a_time_ms": [], "chain_ms": [], "chain_prefetch_ms": []}
    for _ in range(3):
        res["layers_one_at_a_time_ms"].append(sum(timed(g, args.steps) for g in singles))
        res["chain_ms"].append(timed(g_chain, args.steps))
        if g_pref is not None:
            res["chain_prefetch_ms"].append(timed(g_pref, args.steps))
    g_chain.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(bufs[L - 1].y, y_ref))
    if g_pref is not None:
        g_pref.replay()
        torch.cuda.synchronize()
        same = same and bool(torch.equal(bufs[L - 1].y, y_ref))
    best = {k: (float(np.min(v)) if v else None) for k, v in res.items()}
    ms = best["chain_prefetch_ms"] if g_pref is not None else best["chain_ms"]
    line = {"metric": METRIC + f" ({L} chained layers)", "value": base.T / (ms * 1e-3),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": base.dtype,
            "data": "synthetic (seeded N(0,1) inputs, N(0,1/d_in) weights, distinct per layer)",
            "config": {"workload": f"{base.name}x{L}", "T": base.T, "d_model": base.d_model,
                       "n_ffn": base.n_ffn, "n_zero": base.n_zero, "d_ff": base.d_ff,
                       "top_k": base.top_k, "layers": L, "prefetch": bool(args.prefetch)},
            "chain": {**best, "rounds": res, "outputs_equal_eager_chain": same,
                      "per_layer_ms_chain": best["chain_ms"] / L,
                      "per_layer_ms_alone": best["layers_one_at_a_time_ms"] / L}}
    print(json.dumps(line), flush=True)
    if not same:
        sys.exit(1)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    if args.tokens and (args.tokens < 1 or args.workload == "headline" or args.scmoe
                        or args.layers):
        print("bench.py: --tokens takes a positive count and a --workload other than the "
              "default headline run (no --scmoe / --layers)", file=sys.stderr)
        sys.exit(2)
    if args.scmoe:
        if args.workload == "headline":
            args.workload = "decode_bf16"
        return scmoe_main(args)
    if args.layers:
        if args.workload == "headline":
            args.workload = "decode_bf16"
        return chain_main(args)

    import torch

    from sparse_moe_layer_03_amd import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    if args.workload != "headline":
        w = S.WORKLOADS[args.workload]
        if args.tokens:
            import dataclasses

            w = dataclasses.replace(w, T=args.tokens, name=f"{w.name}@T{args.tokens}")
        line = run_workload(w, args, build_model(w, dev), dev)
        print(json.dumps(line), flush=True)
        return

    # prefill line and decode record on the same resident 512-expert weights
    wp, wdec = S.WORKLOADS["prefill_bf16"], S.WORKLOADS["decode_bf16"]
    assert (wp.d_model, wp.n_ffn, wp.n_zero, wp.d_ff, wp.seed) == \
        (wdec.d_model, wdec.n_ffn, wdec.n_zero, wdec.d_ff, wdec.seed)
    mdl = build_model(wp, dev)
    print(f"bench.py: weights resident ({3 * wp.n_ffn * wp.d_model * wp.d_ff * 2 / 1e9:.1f} GB); "
          "timing prefill_bf16", file=sys.stderr, flush=True)
    line = run_workload(wp, args, mdl, dev, cpu=False)
    print("bench.py: timing decode_bf16", file=sys.stderr, flush=True)
    dec = run_workload(wdec, args, mdl, dev, cpu=False)
    if not args.no_cpu_baseline:
        from sparse_moe_layer_03_amd import synth as S2
        for rec, w in ((line, wp), (dec, wdec)):
            print(f"bench.py: CPU oracle baseline, {w.name}", file=sys.stderr, flush=True)
            x = S2.make_x(w, 0, dev)
            v, threads, sample = cpu_baseline_sampled(w, mdl, x)
            rec["cpu_baseline"] = {"value": v, "unit": "tokens/s", "cores": threads,
                                   "kind": "oracle", "cpu": cpu_model(),
                                   "host_cpus": os.cpu_count(), "sample": sample}
    keep = ("value", "unit", "ms_per_step", "config", "roofline", "roofline_down", "layer",
            "step_ms", "stages_ms_mean", "graph", "eager", "ffn_assignments_per_step_mean",
            "touched_ffn_experts_per_step_mean", "cpu_baseline")
    line["decode"] = {k: dec[k] for k in keep}
    line["metric_fracs"] = {
        "prefill_mfma_frac": line["layer"]["mfma_frac"],
        "decode_hbm_frac": dec["layer"]["hbm_frac"],
        "targets": {"prefill_mfma_frac": 0.60, "decode_hbm_frac": 0.70}}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
