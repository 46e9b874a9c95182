"""Summaries of rocprofv3 runs of bench.py, written as short Markdown files.

Input: a directory holding, for each workload N that was profiled,
  kt_cN/run_kernel_stats.csv     rocprofv3 --kernel-trace --stats --output-format csv
  kt_cN.log                      that run's output (the bench JSON line)
  pmc_cN_FETCH_SIZE/run_counter_collection.csv   rocprofv3 --pmc FETCH_SIZE
  pmc_cN_WRITE_SIZE/run_counter_collection.csv   rocprofv3 --pmc WRITE_SIZE
plus pmc_copy_FETCH_SIZE / pmc_copy_WRITE_SIZE of ``bench.py --copy-probe-mib M``
(a plain device copy of M MiB, which reads and writes M MiB) and digest.txt
(build.source_digest() of the profiled sources).

Output: one <kernel>_<workload>.md per workload (kernel-trace statistics next
to the bench line's HIP-event time) and hbm_traffic_counters.md (HBM bytes per
dispatch of each attention kernel, calibrated against the copy, with a JSON
block that bench.py reads).

    python3 -m paged_kv_attention_gather_amd.profile_summary DIR OUT_DIR [--copy-mib 256]
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
from collections import defaultdict

WORKLOADS = {
    2: "decode_int8",
    3: "append_prefill",
    4: "spec_decode",
    5: "mla_decode",
}

KT_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
          "-d $OUT/kt_c{c} -o run -- python3 $R/bench.py --config {c} --steps 10 "
          "--warmup 3 --no-cpu-baseline --no-extra-configs")
PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} --output-format csv "
           "-d $OUT/pmc_c{c}_{ctr} -o run -- python3 $R/bench.py --config {c} --steps 3 "
           "--warmup 1 --no-cpu-baseline --no-extra-configs")
COPY_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} --output-format csv "
            "-d $OUT/pmc_copy_{ctr} -o run -- python3 $R/bench.py --copy-probe-mib {mib}")


def _short(name: str) -> str:
    n = name.replace("(pa::AttnParams)", "").replace("(pa::MergeParams)", "").replace("void ", "")
    return n[:90]


def _bench_line(path):
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("{"):
            return json.loads(line)
    return None


def _counter(path, kernel_prefix):
    """Per-dispatch values of the counter for kernels whose name starts with kernel_prefix."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: v for k, v in vals.items() if _short(k).startswith(kernel_prefix)}


def summarize(root: str, out: str, copy_mib: int) -> None:
    os.makedirs(out, exist_ok=True)
    digest = open(os.path.join(root, "digest.txt")).read().strip()
    copy = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = _counter(os.path.join(root, f"pmc_copy_{ctr}", "run_counter_collection.csv"), "__amd_rocclr_copyBuffer")
        v = [x for k in vals for x in vals[k] if x > 1000]
        copy[ctr] = statistics.median(v)
    copy_kib = copy_mib * 1024
    fetch_factor = round(copy_kib / copy["FETCH_SIZE"], 3)
    write_factor = round(copy_kib / copy["WRITE_SIZE"], 3)

    table = {}
    for c, wname in WORKLOADS.items():
        kt = os.path.join(root, f"kt_c{c}", "run_kernel_stats.csv")
        if not os.path.exists(kt):
            continue
        rows = list(csv.DictReader(open(kt)))
        bench = _bench_line(os.path.join(root, f"kt_c{c}.log"))
        kname = bench["roofline"]["kernel"] if bench else "paged"
        att = [r for r in rows if _short(r["Name"]).startswith("pa::" + kname)]
        lines = [f"# {kname} on {wname} (bench.py --config {c})", "",
                 f"Kernel sources: `{digest}` (build.source_digest()).", "",
                 "Command (R = repository root, OUT = the profile output directory):", "", "```", KT_CMD.format(c=c), "```", "",
                 "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        lines.append("")
        lines.append("(The 1 GiB read of the cache flush before every step and torch's own fills are "
                     "listed too; the profiler adds a few microseconds per launch to tiny kernels.)")
        if bench:
            roof = bench["roofline"]
            avg = float(att[0]["AverageNs"]) / 1e3 if att else float("nan")
            lines += ["", "Same run, bench.py's HIP-event time of the attention kernel (deferred-merge call): "
                      f"**{roof['kernel_ms'] * 1e3:.2f} us** per launch vs rocprofv3 average **{avg:.2f} us**.",
                      "", f"bench line: value {bench['value']} {bench['unit']}, roofline achieved "
                      f"{roof['achieved']} {roof['unit']} of {roof['peak']} (frac {roof['frac']}), "
                      f"chunk_size {bench['config']['chunk_size']}."]
        open(os.path.join(out, f"{kname}_{wname}.md"), "w").write("\n".join(lines) + "\n")

        entry = {"kernel": kname, "chunk_size": bench["config"]["chunk_size"] if bench else None}
        for ctr, key in (("FETCH_SIZE", "fetch_kib_per_dispatch"), ("WRITE_SIZE", "write_kib_per_dispatch")):
            path = os.path.join(root, f"pmc_c{c}_{ctr}", "run_counter_collection.csv")
            if not os.path.exists(path):
                continue
            vals = _counter(path, "pa::" + kname)
            v = [x for k in vals for x in vals[k]]
            entry[key] = round(statistics.mean(v), 1)
            entry[key.replace("per_dispatch", "dispatches")] = len(v)
        if bench:
            entry["alg_bytes_per_launch"] = bench["roofline"].get("alg_bytes_per_launch", bench["config"].get("alg_bytes"))
        table[str(c)] = entry

    lines = ["# HBM traffic of the attention kernels (FETCH_SIZE / WRITE_SIZE)", "",
             f"Kernel sources: `{digest}`.  bench.py reports `roofline.traffic` from the JSON below only "
             "while build.source_digest() still equals this value.", "",
             "Counters are per dispatch, in KiB, averaged over the profiled dispatches of the attention "
             "kernel.  Calibration: a plain device copy of "
             f"{copy_mib} MiB (reads and writes {copy_mib} MiB) reads FETCH_SIZE {copy['FETCH_SIZE']:.0f} KiB "
             f"and WRITE_SIZE {copy['WRITE_SIZE']:.0f} KiB, so HBM bytes = FETCH_SIZE x {fetch_factor} + "
             f"WRITE_SIZE x {write_factor} (KiB).", "",
             "Commands (R = repository root, OUT = the profile output directory), one pass per counter:", "", "```",
             COPY_CMD.format(ctr="FETCH_SIZE", mib=copy_mib), COPY_CMD.format(ctr="WRITE_SIZE", mib=copy_mib)]
    for c in table:
        lines += [PMC_CMD.format(ctr="FETCH_SIZE", c=c), PMC_CMD.format(ctr="WRITE_SIZE", c=c)]
    lines += ["```", "", "| workload | kernel | FETCH KiB | WRITE KiB | HBM bytes / launch | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|---|"]
    for c, e in table.items():
        if "fetch_kib_per_dispatch" not in e or "write_kib_per_dispatch" not in e:
            continue
        hbm = e["fetch_kib_per_dispatch"] * 1024 * fetch_factor + e["write_kib_per_dispatch"] * 1024 * write_factor
        alg = e.get("alg_bytes_per_launch") or 0
        lines.append(f"| {WORKLOADS[int(c)]} | {e['kernel']} | {e['fetch_kib_per_dispatch']} | "
                     f"{e['write_kib_per_dispatch']} | {hbm:.0f} | {alg} | {hbm / alg if alg else float('nan'):.3f} |")
    data = {"source_digest": digest, "fetch_factor": fetch_factor, "write_factor": write_factor,
            "copy_mib": copy_mib, "configs": table}
    lines += ["", "```json", json.dumps(data, indent=1), "```", ""]
    open(os.path.join(out, "hbm_traffic_counters.md"), "w").write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("root")
    ap.add_argument("out")
    ap.add_argument("--copy-mib", type=int, default=256)
    a = ap.parse_args()
    summarize(a.root, a.out, a.copy_mib)


if __name__ == "__main__":
    main()
