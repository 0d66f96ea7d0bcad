#!/usr/bin/env python3
"""Turn rocprofv3 output of bench.py into the short summaries under profiles/.

  python profile_summaries.py trace <stats_dir> <command...>
      <stats_dir> holds a `rocprofv3 --kernel-trace --stats --output-format csv`
      run; writes profiles/kernel_trace_<workload>.md (per-kernel calls and
      average / min / max duration).
  python profile_summaries.py trace-as <workload> <stats_dir> <command...>
      the same for a bench run of another workload (bench.py --prefill-config).
  python profile_summaries.py mfma <pmc_dir> <stats_dir> <command...>
      a `rocprofv3 --pmc MfmaUtil MfmaFlopsF16 MfmaFlopsBF16` run of the bench
      command and a kernel-trace run (for durations); writes
      profiles/mfma_<workload>.json with, per prefill kernel, the counters'
      MFMA busy percentage of all SIMDs and the executed MFMA FLOP per launch
      (including hi/lo splits and one-hot transposes) as TFLOP/s against the
      2.5 PFLOP/s dense fp16/bf16 peak.
  python profile_summaries.py mfma-as <tag> <pmc_dir> <stats_dir> <command...>
      the same for a bench run of another workload, whose fused prefill kernel is
      summarised as profiles/mfma_prefill_chunk_<tag>.json (tag e.g. T35413_H32).
  python profile_summaries.py traffic <fetch_dir> <write_dir> <command...>
      the two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the
      same bench command; writes profiles/traffic_<kernel>.json with the HBM
      bytes per launch of each bench kernel.  Both counters are scaled by
      what they read for the bench's 1 GiB device-to-device copy (the
      __amd_rocclr_copyBuffer dispatches: 2^30 bytes read, 2^30 written).
  python profile_summaries.py traffic-as <tag> <fetch_dir> <write_dir> <command...>
      the same for a bench run of another workload (bench.py --prefill-config):
      profiles/traffic_prefill_chunk_<tag>.json for its fused prefill kernel.

The command that produced the run is passed after the directories and stored
verbatim.  bench.py uses a traffic figure only while its `source_digest`
matches the kernel sources.
"""
import csv
import glob
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
from bench import source_digest  # noqa: E402

WORKLOAD = "prefill_split_T8192_H8_decode_rows4096_f32"
KERNELS = {  # short kernel name -> summary name (the bench workload's kernels)
    "prefill_split_prep": "prefill_split_prep_T8192_H8",
    "prefill_split_window_a": "prefill_split_window_a_T8192_H8",
    "prefill_split_window_c": "prefill_split_window_c_T8192_H8",
    "prefill_split_chain": "prefill_split_chain_T8192_H8",
    "decode_kernel": "decode_f32_rows4096_H8",
    "stream_kernel": "decode_f32_rows4096_H8",   # kda_decode's many-row shape
}
COPY = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def short(name):
    m = re.search(r"(prefill_split_prep|prefill_split_chain|prefill_split_window_a|"
                  r"prefill_split_window_c|prefill_chunk_kernel|"
                  r"prefill_serial_kernel|decode_kernel|stream_kernel|__amd_rocclr_\w+)", name)
    return m.group(1) if m else name[:60]


def one(pattern):
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        sys.exit(f"no file matches {pattern}")
    return hits[0]


def trace(stats_dir, command, workload=WORKLOAD):
    rows = list(csv.DictReader(open(one(os.path.join(stats_dir, "**", "*kernel_stats.csv")))))
    what = "default workload" if workload == WORKLOAD else "workload"
    out = [f"# Kernel trace: bench.py {what} ({workload})", "",
           "Command:", "", "```", command, "```", "",
           "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    out += ["", f"Kernel sources digest: `{source_digest()}`", ""]
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.md")
    open(path, "w").write("\n".join(out))
    print(path)


def per_kernel(pmc_dir, counter):
    path = one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    vals = {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        vals.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]) * 1024.0)
    return vals


def traffic(fetch_dir, write_dir, command, kernels=None):
    kernels = KERNELS if kernels is None else kernels
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    big = lambda xs: [x for x in xs if x > 0.5 * COPY_BYTES]
    f_copy, w_copy = big(fetch.get(COPY, [])), big(write.get(COPY, []))
    if not f_copy or not w_copy:
        sys.exit("the 1 GiB copy dispatches were not found in the counter runs")
    f_scale = COPY_BYTES / (sum(f_copy) / len(f_copy))
    w_scale = COPY_BYTES / (sum(w_copy) / len(w_copy))
    digest = source_digest()
    for k, name in kernels.items():
        if k not in fetch or k not in write:
            continue
        fb = f_scale * sum(fetch[k]) / len(fetch[k])
        wb = w_scale * sum(write[k]) / len(write[k])
        rec = {"kernel": k, "workload": name, "bytes_per_launch": fb + wb,
               "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
               "dispatches": len(fetch[k]), "fetch_scale": f_scale, "write_scale": w_scale,
               "calibration": f"{COPY} of {COPY_BYTES} bytes read and written",
               "source_digest": digest, "command": command}
        path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        json.dump(rec, open(path, "w"), indent=1)
        print(path, f"{(fb + wb) / 1e6:.2f} MB/launch")


def mfma(pmc_dir, stats_dir, command, kernels=None, workload=WORKLOAD):
    kernels = KERNELS if kernels is None else kernels
    path = one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    vals = {}
    for r in csv.DictReader(open(path)):
        k = (short(r["Kernel_Name"]), r["Counter_Name"])
        vals.setdefault(k, {}).setdefault(r["Dispatch_Id"], 0.0)
        vals[k][r["Dispatch_Id"]] += float(r["Counter_Value"])
    avg = lambda d: sum(d.values()) / len(d) if d else 0.0
    dur = {short(r["Name"]): float(r["AverageNs"]) for r in
           csv.DictReader(open(one(os.path.join(stats_dir, "**", "*kernel_stats.csv"))))}
    out = {"workload": workload, "peak_tflops": 2500.0, "source_digest": source_digest(),
           "command": command, "kernels": {}}
    for k in kernels:
        if not k.startswith("prefill") or (k, "MfmaUtil") not in vals:
            continue
        flops = avg(vals.get((k, "MfmaFlopsF16"), {})) + avg(vals.get((k, "MfmaFlopsBF16"), {}))
        ns = dur.get(k)
        out["kernels"][k] = {
            "mfma_busy_pct_of_simds": avg(vals[(k, "MfmaUtil")]),
            "executed_mfma_flop_per_launch": flops,
            "avg_us": ns / 1e3 if ns else None,
            "executed_tflops": flops / ns / 1e3 if ns else None,
            "frac_of_peak": flops / ns / 1e3 / 2500.0 if ns else None}
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}.json")
    json.dump(out, open(path, "w"), indent=1)
    print(path)
    for k, v in out["kernels"].items():
        print(f"  {k:28s} busy {v['mfma_busy_pct_of_simds']:6.2f}%  {v['executed_tflops'] or 0:8.1f} TFLOP/s")


if __name__ == "__main__":
    if len(sys.argv) >= 4 and sys.argv[1] == "trace":
        trace(sys.argv[2], " ".join(sys.argv[3:]))
    elif len(sys.argv) >= 5 and sys.argv[1] == "trace-as":
        trace(sys.argv[3], " ".join(sys.argv[4:]), workload=sys.argv[2])
    elif len(sys.argv) >= 5 and sys.argv[1] == "mfma":
        mfma(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif len(sys.argv) >= 6 and sys.argv[1] == "mfma-as":
        tag = sys.argv[2]
        mfma(sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]),
             kernels={"prefill_chunk_kernel": f"prefill_chunk_{tag}"},
             workload=f"prefill_chunk_{tag}")
    elif len(sys.argv) >= 5 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif len(sys.argv) >= 6 and sys.argv[1] == "traffic-as":
        tag = sys.argv[2]
        traffic(sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]),
                kernels={"prefill_chunk_kernel": f"prefill_chunk_{tag}"})
    else:
        sys.exit(__doc__)
