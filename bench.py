#!/usr/bin/env python3
"""Benchmark of the exact top-k engine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3k64]

A step is one exact top-k call (the whole pipeline: sample, threshold,
filter, refine, fallback checks, output) over one synthetic input already
resident in HBM.  Three input buffers rotate so that no call finds its input
in the 256 MB last-level cache.  Prints one JSON line.

Extra modes (measurement plumbing, not part of the timed line):
    --pmc-run                 a short run for rocprofv3 --pmc: two calibration
                              kernels of known traffic, then a few steps
    --pmc-summary A B [C]     read the rocprofv3 counter CSVs of the FETCH_SIZE
                              run (A), the WRITE_SIZE run (B) and optionally
                              an instruction-mix run (C, SQ counters) of
                              --workload and print the summary for profiles/
    --trace-summary D         per-kernel durations from a rocprofv3 kernel trace
                              of a bench run (directory D) for profiles/
    --calibrate W1,W2,...     measure the whole call over the tuned policy's
                              grid of sample sizes on each workload and fit
                              the cost ratio tau_B / tau_A of Eq. 13
    --balance                 the filter's per-workgroup end times by XCD and
                              slot (workgroup trace), for profiles/
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "top-k Gelem/s and HBM GB/s (% of peak), N=2^28 fp32 k=64, 1 MI355X"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "top_selection_sample_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "topk_part_filter.hpp")   # the filter kernel's source
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30


def traffic_file(workload: str) -> str:
    """The committed rocprofv3 counter summary of one workload."""
    return os.path.join(PROFILES, f"pmc_{workload}.txt")

WORKLOADS = {
    # name: (config, k, description)
    "c3k64": ("c3", 64, "1 row x 2^28 fp32 standard normal, k=64"),
    "c3k16": ("c3", 16, "1 row x 2^28 fp32 standard normal, k=16"),
    "c3k2048": ("c3", 2048, "1 row x 2^28 fp32 standard normal, k=2048"),
    "c4v1": ("c4v1", 64, "128 rows x 2^20 fp32 Pareto(1.5) with random signs, k=64 per row"),
    "c4v2": ("c4v2", 64, "128 rows x 2^20 fp32 Pareto(1.5) rows sorted ascending, k=64 per row"),
    "c4v3": ("c4v3", 64, "128 rows x 2^20 fp32 zeros with 64 ones per row, k=64 per row"),
    "c5": ("c5", 131072, "BatchTopK 4096 x 65536 bf16 ReLU(N(0,1)) flattened, k=131072"),
    "c1": ("c1", 10, "1 row x 4096 int32 uniform [0,1000), k=10"),
    "c2": ("c2", 10, "1 row x 65536 int32 uniform [0,2^24), k=10"),
}


def kernel_source_hash() -> str:
    """Hash of everything the filter kernel is compiled from: the device
    header, the filter's section of the kernel source, and the compile
    flags.  Counter data taken on another version of these is stale."""
    with open(KERNEL_SRC) as f:
        src = f.read()
    a = src.index("// Filter (Prof-K section 3")
    b = src.index("__device__ __forceinline__ void start_exact")
    h = hashlib.sha256()
    with open(os.path.join(CSRC, "topk_device.hpp"), "rb") as f:
        h.update(f.read())
    h.update(src[a:b].encode())
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_tss_build", os.path.join(ROOT, "top_selection_sample_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    h.update(" ".join(mod.FLAGS).encode())
    return h.hexdigest()[:16]


def load_inputs(name: str):
    import numpy as np
    import workloads
    cfg, k, desc = WORKLOADS[name]
    x, dt, _, meta = workloads.config(cfg)
    if cfg == "c5":
        x = x.reshape(1, -1)
    return x, dt, k, desc, meta


def to_device(x, dt):
    import numpy as np
    import torch
    if dt == "bf16":
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def algorithmic_bytes(rows, n, k, es, plan, R_mean):
    """Bytes the method must move per call: one read of the input, the
    sampled elements and their keys, the candidates written and read back,
    and the output."""
    b = rows * n * es
    if plan["path"] == 0:
        b += rows * plan["S"] * (es + 4 + 4)
        b += R_mean * 8 * 2
    b += rows * k * (es + 8)
    return b


def read_traffic(workload):
    """HBM bytes per launch of the filter kernel measured by rocprofv3
    counters, if the committed summary of this workload was taken on the
    current kernel source (else None)."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            kk, vv = line.split(":", 1)
            fields[kk.strip()] = vv.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(x, dt, k, budget_s=12.0, max_calls=5, threads=1):
    """Median seconds of the oracle's selection on the whole workload (inputs
    in host memory): the plain partial sort, or its chunked form on
    `threads` threads."""
    import oracle
    oracle.lib()
    times = []
    t_start = time.time()
    while len(times) < max_calls and (time.time() - t_start) < budget_s:
        t0 = time.perf_counter()
        if threads == 1:
            oracle.topk(x, k, dt)
        else:
            oracle.topk_chunked(x, k, threads, dt)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return med, len(times)


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def fallback_rate(tss, bufs, k, rows, calls, policy, steps=0):
    """Fallback rate and survivors of one parameter policy over `calls` calls
    with fresh seeds; with steps > 0 also the time per call over that many
    calls (fresh seeds, fallbacks included as they come)."""
    import torch
    p = tss.default_params(policy=policy)
    n = bufs[0].shape[1]
    cap = tss.plan(n, rows, k, bufs[0].dtype, params=p)["cap"]
    timed = {}
    if steps:
        tss.topk(bufs[0], k, params=p)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(steps):
            tss.topk(bufs[i % len(bufs)], k, params=p)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        timed = {"ms_per_call_with_fallbacks": round(ms, 4),
                 "gelem_s_with_fallbacks": round(rows * n / (ms * 1e-3) / 1e9, 3)}
    fb = 0
    r_sum = 0
    w_sum = 0
    nrow = 0
    for i in range(calls):
        tss.topk(bufs[i % len(bufs)], k, params=p)
        st = tss.read_stats(rows)
        for r in st:
            fb += 1 if r["path"] == 1 else 0
            r_sum += r["r_sampled"]
            # candidates the filter writes: those above tau, and the ties
            # while the tie region has room
            w_sum += r["r_sampled"] - r["ties"] + min(r["ties"], cap)
            nrow += 1
    return {"calls": calls, "row_selections": nrow, "fallbacks": fb,
            "rate": fb / max(nrow, 1), "mean_R": r_sum / max(nrow, 1),
            "mean_written": w_sum / max(nrow, 1), **timed}


def relaxed_trade(tss, bufs, k, rows, steps, calls, ov, oi, recall=0.95):
    """Relaxed recall (Prof-K abstract and section 1): the same call with the
    parameters chosen for k_eff = ceil(recall * k).  Times K calls, then over
    `calls` calls with fresh seeds counts the rows that kept fewer than k
    (route 3) and the fraction of the true top-k returned (every returned
    index is a true top-k element, so recall = kept slots / k)."""
    import torch
    n = bufs[0].shape[1]
    pr = tss.default_params(recall=recall)
    pl = tss.plan(n, rows, k, bufs[0].dtype, params=pr)
    for i in range(3):
        tss.topk(bufs[i % 3], k, params=pr, out=(ov, oi))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(steps):
        tss.topk(bufs[i % 3], k, params=pr, out=(ov, oi))
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    partial = fallback = 0
    kept = 0
    for i in range(calls):
        tss.topk(bufs[i % 3], k, params=pr, out=(ov, oi))
        st = tss.read_stats(rows)
        partial += sum(1 for r in st if r["path"] == 3)
        fallback += sum(1 for r in st if r["path"] == 1)
        kept += int((oi >= 0).sum().item())
    return {"recall_target": recall, "k_eff": pl["k_eff"], "S": pl["S"], "t": pl["t"],
            "M": pl["M"], "ms_per_step": round(ms, 4), "calls": calls,
            "partial_rows": partial, "fallback_rows": fallback,
            "mean_recall": round(kept / (calls * rows * k), 6)}


def run_bench(args):
    import numpy as np
    import torch
    import top_selection_sample_amd as tss

    x, dt, k, desc, meta = load_inputs(args.workload)
    rows, n = x.shape
    es = 2 if dt == "bf16" else 4
    x0 = to_device(x, dt)
    bufs = [x0]
    for shift in (n // 3 + 1, (2 * n) // 3 + 7):
        bufs.append(torch.roll(x0, shifts=shift, dims=1).contiguous())
    torch.cuda.synchronize()
    ov = torch.empty((rows, k), dtype=x0.dtype, device="cuda")
    oi = torch.empty((rows, k), dtype=torch.int64, device="cuda")
    plan = tss.plan(n, rows, k, dt)

    for i in range(args.warmup):
        tss.topk(bufs[i % 3], k, out=(ov, oi))
    torch.cuda.synchronize()

    # timed region: K whole calls
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        tss.topk(bufs[i % 3], k, out=(ov, oi))
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps

    # the same K calls captured in one HIP graph (own workspace, sized by
    # eager calls first) and replayed: what remains without host launches
    gws = tss.Workspace()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            tss.topk(bufs[i % 3], k, workspace=gws, out=(ov, oi))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            tss.topk(bufs[i % 3], k, workspace=gws, out=(ov, oi))
    graph.replay()
    torch.cuda.synchronize()
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    graph_replay = {"ms_per_step": round(ev0.elapsed_time(ev1) / args.steps, 4),
                    "calls_per_graph": args.steps}
    del graph, gws

    # stage timing: HIP events on the launch stream around each stage
    tss.profile_enable(True)
    tss.profile_read()
    ev0.record()
    for i in range(args.steps):
        tss.topk(bufs[i % 3], k, out=(ov, oi))
    ev1.record()
    torch.cuda.synchronize()
    stages = tss.profile_read()
    tss.profile_enable(False)
    ms_step_profiled = ev0.elapsed_time(ev1) / args.steps

    # fallback rate and mean survivors per parameter policy (fresh seeds)
    fb_calls = args.fallback_calls or (1000 if rows == 1 else 100)
    fb = {"tuned": fallback_rate(tss, bufs, k, rows, fb_calls, tss.POLICY_TUNED)}
    if plan["path"] == 0:
        fb["exact_tail"] = fallback_rate(tss, bufs, k, rows, fb_calls, tss.POLICY_EXACT_TAIL,
                                         args.steps)
        fb["alg1"] = fallback_rate(tss, bufs, k, rows, fb_calls, tss.POLICY_ALG1, args.steps)
    R_mean = fb["tuned"]["mean_written"] * rows

    # cost of one fallback: the exact route over the whole input
    exact_ms = None
    if plan["path"] == 0:
        pe = tss.default_params(force_path=tss.PATH_EXACT)
        tss.topk(bufs[0], k, params=pe, out=(ov, oi))
        torch.cuda.synchronize()
        ev0.record()
        for i in range(5):
            tss.topk(bufs[i % 3], k, params=pe, out=(ov, oi))
        ev1.record()
        torch.cuda.synchronize()
        exact_ms = ev0.elapsed_time(ev1) / 5

    # relaxed recall: the accuracy-speed trade at a 95% target
    relaxed = None
    if plan["path"] == 0:
        relaxed = relaxed_trade(tss, bufs, k, rows, args.steps, min(fb_calls, 200), ov, oi)
        relaxed["speedup"] = round(ms_step / relaxed["ms_per_step"], 4)
        relaxed["plan_changed"] = (relaxed["S"], relaxed["t"], relaxed["M"]) != (
            plan["S"], plan["t"], plan["M"])

    # read ceiling: the same input read once per launch with the filter's
    # access pattern and nothing else (k_stream_read), same K
    ceiling = None
    if plan["path"] == 0:
        sink = torch.zeros(64, dtype=torch.int32, device="cuda")
        for i in range(3):
            tss.stream_read(bufs[i % 3], sink)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            tss.stream_read(bufs[i % 3], sink)
        ev1.record()
        torch.cuda.synchronize()
        t_read = ev0.elapsed_time(ev1) / args.steps * 1e-3
        read_bytes = rows * n * es
        ceiling = {"kernel": "k_stream_read", "unit": "GB/s",
                   "achieved": round(read_bytes / t_read / 1e9, 1),
                   "avg_launch_us": round(t_read * 1e6, 2), "bytes_per_launch": int(read_bytes)}

    # BatchTopK consumer (c5): the selection turned into the sparse
    # activation (zero fill of the [B, d] output, then the K winners written
    # back), alone and after the top-k in one step
    consumer = None
    if args.workload == "c5":
        dense = torch.empty((rows, n), dtype=x0.dtype, device="cuda")
        for i in range(3):
            tss.scatter(ov, oi, n, out=dense)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(args.steps):
            tss.scatter(ov, oi, n, out=dense)
        ev1.record()
        torch.cuda.synchronize()
        t_cons = ev0.elapsed_time(ev1) / args.steps * 1e-3
        ev0.record()
        for i in range(args.steps):
            tss.topk(bufs[i % 3], k, out=(ov, oi))
            tss.scatter(ov, oi, n, out=dense)
        ev1.record()
        torch.cuda.synchronize()
        t_both = ev0.elapsed_time(ev1) / args.steps * 1e-3
        cbytes = rows * n * es + rows * k * (es + 8) + rows * k * es
        consumer = {"kernels": "k_fill_zero + k_scatter_winners", "bound": "hbm", "unit": "GB/s",
                    "avg_us": round(t_cons * 1e6, 2),
                    "achieved": round(cbytes / t_cons / 1e9, 1), "peak": HBM_PEAK_GBS,
                    "frac": round(cbytes / t_cons / 1e9 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": int(cbytes),
                    "batchtopk_ms_per_step": round(t_both * 1e3, 4)}
        del dense

    elems = rows * n
    gelem_s = elems / (ms_step * 1e-3) / 1e9
    alg_bytes = algorithmic_bytes(rows, n, k, es, plan, R_mean)
    e2e_gbs = alg_bytes / (ms_step * 1e-3) / 1e9

    roof = None
    if plan["path"] == 0 and stages["filter"]["count"]:
        t_filter = stages["filter"]["ms"] / stages["filter"]["count"] * 1e-3
        filt_bytes = elems * es + R_mean * 8
        achieved = filt_bytes / t_filter / 1e9
        traffic = read_traffic(args.workload)
        # (tau from the merge of sorted lists: the filter instantiation that
        # loads a third step before tau)
        tss.topk(bufs[0], k, out=(ov, oi))
        merge = tss.read_stats(rows)[0]["tau_route"] == tss.TAU_FILTER_MERGE
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "k_filter_ahead3" if merge else "k_filter",
                "avg_launch_us": round(t_filter * 1e6, 2),
                "algorithmic_bytes_per_launch": int(filt_bytes)}
        if ceiling:
            ceiling["filter_frac_of_ceiling"] = round(achieved / ceiling["achieved"], 4)

    cpu = cpu_chunked = None
    if not args.no_cpu_baseline:
        med, calls = cpu_baseline(x, dt, k)
        cpu = {"value": round(elems / med / 1e9, 4), "unit": "Gelem/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the full workload ({desc}); {calls} oracle calls, median "
                         f"{med:.2f} s each, single-threaded partial sort on {cpu_model()} "
                         f"({os.cpu_count()} logical CPUs on the host)"}
        # the same on every core the process may use (at most 16)
        T = max(1, min(len(os.sched_getaffinity(0)), 16))
        med, calls = cpu_baseline(x, dt, k, threads=T)
        cpu_chunked = {"value": round(elems / med / 1e9, 4), "unit": "Gelem/s", "cores": T,
                       "kind": "oracle",
                       "sample": f"the full workload; {calls} calls, median {med:.3f} s each, "
                                 f"{T} threads each taking a contiguous chunk of the row and "
                                 f"keeping its own top-k, then one partial sort of the union"}

    stage_ms = {name: round(v["ms"] / v["count"], 4) if v["count"] else None
                for name, v in stages.items()}
    line = {
        "metric": METRIC, "value": round(gelem_s, 3), "unit": "Gelem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dt == "bf16" else ("i32" if dt == "int32" else "f32"),
        "data": "synthetic",
        "config": {"workload": desc, "rows": rows, "n": n, "k": k, "input_dtype": dt,
                   "seed": meta["seed"], "policy": "tuned", "S": plan["S"],
                   "t": plan["t"], "M": plan["M"], "route": ["sampled", "exact", "exact_small"][plan["path"]]},
        "hbm_gbs": round(e2e_gbs, 1), "hbm_frac": round(e2e_gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(alg_bytes),
        "roofline": roof,
        "read_ceiling": ceiling,
        "batchtopk_consumer": consumer,
        "relaxed_recall": relaxed,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_chunked,
        "fallback": fb,
        "exact_route_ms_per_call": round(exact_ms, 4) if exact_ms is not None else None,
        "stage_ms": stage_ms,
        "ms_per_step_with_stage_events": round(ms_step_profiled, 4),
        "graph_replay": graph_replay,
    }
    print(json.dumps(line), flush=True)


def pmc_run(args):
    """Short program for rocprofv3 --pmc.  Two calibration kernels of known
    traffic come first: k_stream_read reads COPY_BYTES with the filter's own
    load pattern (16-byte nontemporal loads; FETCH_SIZE calibration), and a
    plain copy writes COPY_BYTES (WRITE_SIZE calibration).  Then a few
    steps of the workload."""
    import torch
    import top_selection_sample_amd as tss
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    tss.stream_read(src, sink)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    x, dt, k, desc, meta = load_inputs(args.workload)
    xd = to_device(x, dt)
    ov = torch.empty((x.shape[0], k), dtype=xd.dtype, device="cuda")
    oi = torch.empty((x.shape[0], k), dtype=torch.int64, device="cuda")
    for _ in range(max(args.steps, 1)):
        tss.topk(xd, k, out=(ov, oi))
    torch.cuda.synchronize()
    print("pmc run done", flush=True)


def _rows_of(path_glob, counter):
    """(dispatch id, kernel name, value) of every row of a rocprofv3 counter
    CSV for one counter, in dispatch order."""
    out = []
    for f in glob.glob(path_glob, recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter:
                    did = int(row.get("Dispatch_Id") or row.get("Correlation_Id") or 0)
                    out.append((did, row.get("Kernel_Name", ""), float(row["Counter_Value"])))
    out.sort()
    return out


def _short(name: str) -> str:
    """A kernel's name without its return type and argument list
    (tk::k_filter<1>)."""
    nm = name.split("(")[0].strip()
    return nm[5:] if nm.startswith("void ") else nm


def pmc_summary(args):
    """The traffic summary of one workload from the FETCH_SIZE run (A) and
    the WRITE_SIZE run (B): each counter (KiB per dispatch) scaled by what
    it reads for its calibration kernel, per kernel of the pipeline (median
    over its dispatches)."""
    if len(args.pmc_summary) not in (2, 3):
        raise SystemExit("--pmc-summary takes FETCH_DIR WRITE_DIR [SQ_DIR]")
    fetch_dir, write_dir = args.pmc_summary[:2]
    sq_dir = args.pmc_summary[2] if len(args.pmc_summary) == 3 else None
    fe = _rows_of(os.path.join(fetch_dir, "**", "*counter_collection.csv"), "FETCH_SIZE")
    wr = _rows_of(os.path.join(write_dir, "**", "*counter_collection.csv"), "WRITE_SIZE")
    kib = 1024.0

    def first(rows, pred):
        for _, name, v in rows:
            if pred(name):
                return v, _short(name)
        return None, None

    cf, cf_name = first(fe, lambda nm: "k_stream_read" in nm)
    cw, cw_name = first(wr, lambda nm: "copy" in nm.lower())
    scale_f = COPY_BYTES / (cf * kib) if cf else None
    scale_w = COPY_BYTES / (cw * kib) if cw else None
    # the pipeline's kernels: everything after the calibration dispatches
    # (and the input upload's own copies) whose name is one of the library's
    per = {}
    for rows, key in ((fe, "f"), (wr, "w")):
        for _, name, v in rows:
            nm = _short(name)
            if not nm.startswith("tk::") or "k_stream_read" in nm:
                continue
            per.setdefault(nm, {"f": [], "w": []})[key].append(v)
    cfg, k, desc = WORKLOADS[args.workload]
    lines = [
        f"rocprofv3 counter summary: workload {args.workload} ({desc})",
        "",
        "Commands (from /tmp with TMPDIR=/tmp; REPO = repository root, OUT = output dirs):",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT_F -o run -- python3 REPO/bench.py --pmc-run --workload {args.workload} --steps 3",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT_W -o run -- python3 REPO/bench.py --pmc-run --workload {args.workload} --steps 3",
        f"  python3 REPO/bench.py --pmc-summary OUT_F OUT_W --workload {args.workload}",
        "",
        "FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by what it",
        "reads for a kernel of known traffic in the same run: k_stream_read",
        f"(reads {COPY_BYTES} bytes with the filter's load pattern) and a plain copy",
        f"(writes {COPY_BYTES} bytes).",
        "",
        f"kernel_source_sha256_16: {kernel_source_hash()}",
        f"calibration_fetch_kernel: {cf_name}",
        f"calibration_write_kernel: {cw_name}",
        f"fetch_kib_calibration: {cf}",
        f"write_kib_calibration: {cw}",
        f"scale_fetch: {scale_f}",
        f"scale_write: {scale_w}",
        "",
        "| kernel | dispatches | FETCH KiB (median) | WRITE KiB (median) | HBM read bytes | HBM write bytes |",
        "|---|---|---|---|---|---|",
    ]
    filt = None
    for nm in sorted(per):
        fv, wv = sorted(per[nm]["f"]), sorted(per[nm]["w"])
        fm = fv[len(fv) // 2] if fv else None
        wm = wv[len(wv) // 2] if wv else None
        fb = fm * kib * scale_f if fm is not None and scale_f else None
        wb = wm * kib * scale_w if wm is not None and scale_w else None
        lines.append(f"| {nm} | {len(fv)} | {fm} | {wm} | "
                     f"{'' if fb is None else f'{fb:.0f}'} | {'' if wb is None else f'{wb:.0f}'} |")
        if "k_filter" in nm and fb is not None and wb is not None:
            filt = (fb, wb)
    lines.append("")
    if filt:
        lines.append(f"k_filter_fetch_bytes_scaled: {filt[0]:.0f}")
        lines.append(f"k_filter_write_bytes_scaled: {filt[1]:.0f}")
        lines.append(f"hbm_bytes_per_launch: {filt[0] + filt[1]:.0f}")
    if sq_dir:
        lines += [""] + sq_table(sq_dir, args.workload)
    print("\n".join(lines))


def trace_summary(args):
    """Per-kernel durations of the top-k calls of one bench run under
    rocprofv3 --kernel-trace (the CSV under TRACE_DIR): the warm-up, timed
    and first graph-replayed calls, all on the default plan.  A call starts
    at its first kernel (the sampler, a caller-given threshold's set-up, the
    exact route's set-up or the one-workgroup route)."""
    files = glob.glob(os.path.join(args.trace_summary, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {args.trace_summary}")
    with open(files[0]) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Dispatch_Id"]))
    ks = [(_short(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    ks = [k for k in ks if k[0].startswith("tk::") and "k_stream_read" not in k[0]]
    firsts = ("tk::k_sample", "tk::k_force_tau", "tk::k_setup_exact", "tk::k_exact_small")
    starts = [i for i, k in enumerate(ks) if k[0].startswith(firsts)]
    calls = [ks[s:(starts[j + 1] if j + 1 < len(starts) else len(ks))] for j, s in enumerate(starts)]
    sel = calls[:args.warmup + 2 * args.steps]
    per, spans = {}, []
    for c in sel:
        spans.append((c[-1][2] - c[0][1]) / 1e3)
        for name, a, b in c:
            per.setdefault(name, []).append((b - a) / 1e3)
    cfg, k, desc = WORKLOADS[args.workload]
    out = [f"rocprofv3 kernel trace, workload {args.workload}: {desc}", "",
           "Commands (run from /tmp with TMPDIR=/tmp; REPO = the repository root):",
           f"  rocprofv3 --kernel-trace --stats --output-format csv -d OUT -o run -- python3 REPO/bench.py "
           f"--steps {args.steps} --warmup {args.warmup} --workload {args.workload} --no-cpu-baseline "
           f"--fallback-calls 3",
           f"  python3 REPO/bench.py --trace-summary OUT --steps {args.steps} --warmup {args.warmup} "
           f"--workload {args.workload}", "",
           f"kernel_source_sha256_16: {kernel_source_hash()}", "",
           f"Statistics over the first {len(sel)} top-k calls of that run (warm-up, timed and "
           "graph-replayed calls: the default plan); the later calls of the run (stage timing, "
           "fallback-rate policies, forced exact route) are left out.", "",
           "| kernel | launches | avg us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {name} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                   f"{min(v):.2f} | {max(v):.2f} |")
    if spans:
        out.append(f"| whole call (first kernel start to last kernel end) | {len(spans)} | "
                   f"{statistics.mean(spans):.2f} | {statistics.median(spans):.2f} | "
                   f"{min(spans):.2f} | {max(spans):.2f} |")
    print("\n".join(out))


SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_BRANCH",
               "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU")


def sq_table(sq_dir, workload):
    """Instruction mix per pipeline kernel from one rocprofv3 run of the eight
    SQ counters above (medians over the kernel's dispatches); per wave: the
    counter divided by SQ_WAVES."""
    pat = os.path.join(sq_dir, "**", "*counter_collection.csv")
    med = {}
    for c in SQ_COUNTERS:
        per = {}
        for _, name, v in _rows_of(pat, c):
            nm = _short(name)
            if nm.startswith("tk::") and "k_stream_read" not in nm:
                per.setdefault(nm, []).append(v)
        for nm, vs in per.items():
            vs = sorted(vs)
            med.setdefault(nm, {})[c] = vs[len(vs) // 2]
    out = [
        "Instruction mix (one more run, the same program:",
        f"  rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d OUT_SQ -o run -- "
        f"python3 REPO/bench.py --pmc-run --workload {workload} --steps 3",
        f"  python3 REPO/bench.py --pmc-summary OUT_F OUT_W OUT_SQ --workload {workload})",
        "",
        "| kernel | waves | VALU / wave | SALU / wave | LDS / wave | branch / wave | ACTIVE_INST_VALU / BUSY_CYCLES |",
        "|---|---|---|---|---|---|---|",
    ]
    for nm in sorted(med):
        m = med[nm]
        wv = m.get("SQ_WAVES") or 0.0

        def per(c):
            return f"{m[c] / wv:.1f}" if wv and c in m else ""
        act = (f"{m['SQ_ACTIVE_INST_VALU'] / m['SQ_BUSY_CYCLES']:.3f}"
               if m.get("SQ_BUSY_CYCLES") and "SQ_ACTIVE_INST_VALU" in m else "")
        out.append(f"| {nm} | {wv:.0f} | {per('SQ_INSTS_VALU')} | {per('SQ_INSTS_SALU')} | "
                   f"{per('SQ_INSTS_LDS')} | {per('SQ_INSTS_BRANCH')} | {act} |")
    return out


def calibrate(args):
    """Cost-ratio calibration for the tuned policy (Prof-K section 4,
    "Optimal Sample Size": tau_B / tau_A estimated by microbenchmark).

    For each workload, the mean whole-call time is measured at every sample
    size of the policy's grid (t and M from the exact tail at that S).  Then,
    for each candidate ratio, the policy's choice of S is looked up in the
    measurements; the ratio whose choices lose the least time against the
    best measured S (summed relative excess over the workloads) is
    reported."""
    import math
    import torch
    import top_selection_sample_amd as tss
    d0 = tss.default_params()
    names = args.calibrate.split(",")
    meas = {}
    for name in names:
        x, dt, k, desc, meta = load_inputs(name)
        rows, n = x.shape
        x0 = to_device(x, dt)
        del x
        bufs = [x0] + [torch.roll(x0, shifts=s, dims=1).contiguous()
                       for s in (n // 3 + 1, (2 * n) // 3 + 7)]
        ov = torch.empty((rows, k), dtype=x0.dtype, device="cuda")
        oi = torch.empty((rows, k), dtype=torch.int64, device="cuda")
        grid, j = [], 0
        s_hi = min(d0.s_max, n // 8)
        while True:
            S = int(round(d0.tuned_s_min * 2.0 ** (0.25 * j)))
            if S > s_hi:
                break
            if not grid or S != grid[-1]:
                grid.append(S)
            j += 1
        times = {}
        for S in grid:
            p = tss.default_params(S=S)
            for i in range(3):
                tss.topk(bufs[i % 3], k, params=p, out=(ov, oi))
            torch.cuda.synchronize()
            # mean over many calls with fresh seeds: the occasional fallback
            # is part of the cost being minimised
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(150):
                tss.topk(bufs[i % 3], k, params=p, out=(ov, oi))
            e1.record()
            torch.cuda.synchronize()
            times[S] = e0.elapsed_time(e1) / 150
            pl = tss.plan(n, rows, k, dt, params=p)
            print(f"{name} S={S} t={pl['t']} M={pl['M']} us={times[S] * 1e3:.1f}", flush=True)
        meas[name] = (n, rows, k, dt, times)
        del bufs, x0, ov, oi
        torch.cuda.empty_cache()
    # the two refines (k <= 4096 in one workgroup, larger k by the bucket
    # sort) have their own ratio, and so do batches of small-k rows, whose
    # samples are gathered together: fit each on its own workloads
    ratios = [10 ** (e / 8.0) for e in range(-24, 9)]

    def group_of(v):
        n, rows, k = v[0], v[1], v[2]
        if k > 4096:
            return "tuned_ratio_large"
        return "tuned_ratio_batched" if rows >= d0.tuned_batch_rows else "tuned_ratio"

    for group, field in (("k <= 4096, fewer rows", "tuned_ratio"),
                         (f"k <= 4096, {d0.tuned_batch_rows} rows or more", "tuned_ratio_batched"),
                         ("k > 4096", "tuned_ratio_large")):
        names_g = [nm for nm, v in meas.items() if group_of(v) == field]
        if not names_g:
            continue
        table = []
        for rho in ratios:
            loss = 0.0
            picks = {}
            for name in names_g:
                n, rows, k, dt, times = meas[name]
                S = tss.plan(n, rows, k, dt, params=tss.default_params(**{field: rho}))["S"]
                picks[name] = S
                loss += times[S] / min(times.values()) - 1.0
            table.append((loss, rho, picks))
            print(f"{field} {rho:.4g}: excess {loss * 100:.2f}% picks {picks}", flush=True)
        best = min(l for l, _, _ in table)
        good = [rho for l, rho, _ in table if l <= best + 1e-12]
        print(f"{group}: best excess {best * 100:.2f}% for {field} {min(good):.4g} .. "
              f"{max(good):.4g}; geometric middle {math.sqrt(min(good) * max(good)):.4g}")
    for name, (n, rows, k, dt, times) in meas.items():
        sb = min(times, key=times.get)
        print(f"{name}: best measured S={sb} ({times[sb] * 1e3:.1f} us)")


def balance(args):
    """Filter workgroup balance (the table for profiles/): per-workgroup
    realtime stamps (topk_filter_trace) of the workload's filter over
    rotating inputs.  Per XCD (workgroup l runs on XCD l mod 8) and slot
    (first or second workgroup on its compute unit): the mean end of the scan
    relative to the call's median end, and the group's rate (the inverse of
    its mean time to the end of its scan) relative to the mean rate; then the
    spread of end times and the filter's span (first start to last end)."""
    import numpy as np
    import torch
    import top_selection_sample_amd as tss

    x, dt, k, desc, meta = load_inputs(args.workload)
    rows, n = x.shape
    es = 2 if dt == "bf16" else 4
    x0 = to_device(x, dt)
    bufs = [x0] + [torch.roll(x0, shifts=sh, dims=1).contiguous()
                   for sh in (n // 3 + 1, (2 * n) // 3 + 7)]
    ov = torch.empty((rows, k), dtype=x0.dtype, device="cuda")
    oi = torch.empty((rows, k), dtype=torch.int64, device="cuda")
    plan = tss.plan(n, rows, k, dt)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    trace = torch.zeros(2 * 8192, dtype=torch.int64, device="cuda")
    for i in range(3):
        tss.topk(bufs[i % 3], k, out=(ov, oi))
    tss.filter_trace(trace)
    ends, durs, spans, nwg = [], [], [], None
    for i in range(args.steps):
        trace.zero_()
        tss.topk(bufs[i % 3], k, out=(ov, oi))
        torch.cuda.synchronize()
        t = trace.cpu().numpy().reshape(-1, 2)
        if nwg is None:
            nwg = int(np.count_nonzero(t[:, 0]))
        t = t[:nwg].astype(np.int64)
        t0 = t[:, 0].min()
        ends.append((t[:, 1] - t0) / 100.0)
        durs.append((t[:, 1] - t[:, 0]) / 100.0)
        spans.append((t[:, 1].max() - t0) / 100.0)
    tss.filter_trace(None)
    E, D = np.array(ends), np.array(durs)
    l = np.arange(nwg)
    two = nwg > cus
    groups = [(g, s) for s in ((0, 1) if two else (0,)) for g in range(8)]
    gbytes = rows * n * es
    print(f"# Filter workgroup balance: {desc}")
    print()
    print("Command (REPO = the repository root):")
    print(f"  python3 REPO/bench.py --balance --workload {args.workload} --steps {args.steps}")
    print()
    print(f"Plan: S={plan['S']} t={plan['t']} M={plan['M']}; {nwg} filter workgroups "
          f"({'two' if two else 'one'} per compute unit, {cus} units), equal slices; "
          f"{args.steps} calls on three rotating inputs.  Stamps: the device's 100 MHz realtime "
          f"counter at each workgroup's start and at the end of its scan.")
    print()
    span = float(np.mean(spans))
    print("| filter span (first start to last end) | end spread (max - min) | last end - median end | input / span |")
    print("|---|---|---|---|")
    print(f"| {span:.1f} us | {np.mean(E.max(1) - E.min(1)):.1f} us | "
          f"{np.mean(E.max(1) - np.median(E, axis=1)):.1f} us | {gbytes / span / 1e3:.0f} GB/s |")
    print()
    print("Per group (XCD = workgroup index mod 8; slot b = the second workgroup on its unit): "
          "mean end relative to the call's median end, and the group's rate (1 / mean time to "
          "the end of its scan) relative to the mean rate, parts per 1024.")
    print()
    print("| group | end - median us | rate (/1024) |")
    print("|---|---|---|")
    rates = {}
    for g in groups:
        mk = (l % 8 == g[0]) & ((l >= cus) == bool(g[1]))
        rates[g] = (float(np.mean(E[:, mk].mean(1) - np.median(E, axis=1))), 1.0 / D[:, mk].mean())
    mr = np.mean([r for _, r in rates.values()])
    for g in groups:
        print(f"| {g[0]}{'b' if g[1] else 'a'} | {rates[g][0]:+.1f} | {rates[g][1] / mr * 1024:.0f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3k64", choices=sorted(WORKLOADS))
    ap.add_argument("--fallback-calls", type=int, default=0,
                    help="calls per policy for the fallback rate (default 1000, or 100 for batched rows)")
    ap.add_argument("--calibrate", metavar="WORKLOADS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-run", action="store_true")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR [SQ_DIR]")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR")
    ap.add_argument("--balance", action="store_true",
                    help="filter workgroup balance table (per-workgroup trace), for profiles/")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.gpus != 1:
        print("bench.py: this engine runs on one GPU; --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("1", ""):
        print("bench.py: multi-rank launch is not supported (one GPU only)", file=sys.stderr)
        sys.exit(2)
    if args.pmc_run:
        pmc_run(args)
        return
    if args.calibrate:
        calibrate(args)
        return
    if args.balance:
        balance(args)
        return
    run_bench(args)


if __name__ == "__main__":
    main()
