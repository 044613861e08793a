"""bench.py's command line without a GPU: more than one GPU is refused with a
message, and a multi-rank launch likewise."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_multi_rank_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run([], env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr



def test_pmc_summary_scales_each_kernel(tmp_path):
    # synthetic rocprofv3 counter CSVs: the calibration kernels read / write
    # 2^30 bytes and report half / all of it; the pipeline's kernels report
    # their own KiB.  The summary scales each by its calibration.
    import csv
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch = [(1, "tk::k_stream_read(uint4 const*, unsigned long, unsigned int*)", 524288.0),
             (2, "__amd_rocclr_copyBuffer", 524288.0),
             (3, "void tk::k_sample<1>(...)", 100.0), (4, "void tk::k_filter<1>(...)", 524300.0),
             (5, "void tk::k_sample<1>(...)", 102.0), (6, "void tk::k_filter<1>(...)", 524310.0),
             (7, "void tk::k_filter<1>(...)", 524320.0)]
    write = [(1, "tk::k_stream_read(uint4 const*, unsigned long, unsigned int*)", 0.0),
             (2, "__amd_rocclr_copyBuffer", 1048576.0),
             (3, "void tk::k_sample<1>(...)", 8.0), (4, "void tk::k_filter<1>(...)", 90.0),
             (6, "void tk::k_filter<1>(...)", 92.0), (7, "void tk::k_filter<1>(...)", 94.0)]
    for name, rows, counter in (("f", fetch, "FETCH_SIZE"), ("w", write, "WRITE_SIZE")):
        d = tmp_path / name / "host"
        d.mkdir(parents=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as fh:
            wr = csv.DictWriter(fh, fieldnames=fields)
            wr.writeheader()
            for did, kn, v in rows:
                wr.writerow({"Dispatch_Id": did, "Kernel_Name": kn, "Counter_Name": counter,
                             "Counter_Value": v})
    r = _run(["--pmc-summary", str(tmp_path / "f"), str(tmp_path / "w"), "--workload", "c3k64"])
    assert r.returncode == 0, r.stderr
    out = dict(line.split(":", 1) for line in r.stdout.splitlines() if ": " in line and "|" not in line)
    assert float(out["scale_fetch"]) == 2.0 and float(out["scale_write"]) == 1.0
    assert "tk::k_stream_read" in out["calibration_fetch_kernel"]
    # filter medians: 524310 KiB fetched (x2), 92 KiB written (x1)
    assert int(out["k_filter_fetch_bytes_scaled"]) == 524310 * 1024 * 2
    assert int(out["k_filter_write_bytes_scaled"]) == 92 * 1024
    assert int(out["hbm_bytes_per_launch"]) == 524310 * 2048 + 92 * 1024
    assert "| tk::k_sample<1> | 2 |" in r.stdout


def test_pmc_summary_instruction_mix(tmp_path):
    # a third directory of SQ counters adds per-wave instruction counts
    import csv
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    fixed = [(1, "tk::k_stream_read(uint4 const*)", "FETCH_SIZE", 524288.0),
             (2, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)]
    sq = []
    for did, waves, valu in ((3, 100.0, 26400.0), (5, 100.0, 26600.0), (7, 100.0, 26500.0)):
        for c, v in (("SQ_WAVES", waves), ("SQ_INSTS_VALU", valu), ("SQ_INSTS_SALU", 500.0),
                     ("SQ_INSTS_LDS", 300.0), ("SQ_INSTS_BRANCH", 200.0),
                     ("SQ_WAVE_CYCLES", 9.0e5), ("SQ_BUSY_CYCLES", 1000.0),
                     ("SQ_ACTIVE_INST_VALU", 250.0)):
            sq.append((did, "void tk::k_filter<2>(...)", c, v))
    for name, rows in (("f", fixed[:1]), ("w", fixed[1:]), ("q", sq)):
        d = tmp_path / name
        d.mkdir(parents=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as fh:
            wr = csv.DictWriter(fh, fieldnames=fields)
            wr.writeheader()
            for did, kn, c, v in rows:
                wr.writerow({"Dispatch_Id": did, "Kernel_Name": kn, "Counter_Name": c,
                             "Counter_Value": v})
    r = _run(["--pmc-summary", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "q"),
              "--workload", "c5"])
    assert r.returncode == 0, r.stderr
    # medians: 100 waves, 26500 VALU -> 265.0 per wave; 250 / 1000 busy
    assert "| tk::k_filter<2> | 100 | 265.0 | 5.0 | 3.0 | 2.0 | 0.250 |" in r.stdout


def test_trace_summary_splits_calls(tmp_path):
    # two calls of three kernels each (sample, filter, finish), then a
    # third call beyond warm-up + 2 x steps that must be left out
    import csv
    d = tmp_path / "t" / "host"
    d.mkdir(parents=True)
    rows, did, t = [], 0, 1000
    for call in range(3):
        for kn, dur in (("void tk::k_sample<1>(...)", 5000), ("void tk::k_filter<1>(...)", 150000 + call),
                        ("void tk::k_finish<1>(...)", 10000)):
            did += 1
            rows.append({"Dispatch_Id": did, "Kernel_Name": kn, "Start_Timestamp": t,
                         "End_Timestamp": t + dur})
            t += dur + 1000
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)
    r = _run(["--trace-summary", str(tmp_path / "t"), "--steps", "1", "--warmup", "0",
              "--workload", "c3k64"])
    assert r.returncode == 0, r.stderr
    assert "| tk::k_filter<1> | 2 | 150.00 | 150.00 | 150.00 | 150.00 |" in r.stdout
    assert "| tk::k_sample<1> | 2 | 5.00 | 5.00 | 5.00 | 5.00 |" in r.stdout
    # whole call: 5 + 1 + 150 + 1 + 10 us
    assert "| whole call (first kernel start to last kernel end) | 2 | 167.00" in r.stdout
