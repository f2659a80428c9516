"""Summaries of rocprofv3 runs of bench.py: kernel durations and HBM bytes.

Three runs per workload, each with the program straight after ``--``::

  rocprofv3 --kernel-trace --stats --output-format csv -d T -o run -- \\
      python3 bench.py --config C --steps 50 --warmup 10 --cpu-budget 0
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d F -o run -- \\
      python3 bench.py --config C --steps 5 --warmup 1 --cpu-budget 0 --copy-calibration
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d W -o run -- \\
      python3 bench.py --config C --steps 5 --warmup 1 --cpu-budget 0 --copy-calibration

``python -m paged_kv_cache_18_amd.profiling --config C --trace T --fetch F
--write W --bench-json B`` then writes ``profiles/<kernel>_C.md`` and the
workload's entry of ``profiles/hbm_traffic.json``.  FETCH_SIZE and WRITE_SIZE
(KiB per dispatch) are scaled by what they read for the 1 GiB device copy of
``--copy-calibration`` in the same run.  bench.py reports the scaled bytes per
decode launch as ``roofline.traffic`` only while the sources the counters were
taken from are unchanged (``source_hash``).
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_JSON = os.path.join(PROFILES, "hbm_traffic.json")
COPY_BYTES = 1 << 30


# the files that decide the timed kernels' code and launch configuration
# (other kernels do not change their counters)
HASHED = ["build.py", "csrc/pa_capi.cpp", "csrc/kernels/common.hpp", "csrc/kernels/launch.hpp",
          "csrc/kernels/decode_common.hpp", "csrc/kernels/decode_mfma.hip",
          "csrc/kernels/decode_quant.hip", "csrc/kernels/decode_generic.hip",
          "csrc/kernels/prefill_tile.hip"]


def source_hash():
    """sha256 over the sources of the timed kernels and their launch."""
    h = hashlib.sha256()
    for rel in HASHED:
        h.update(rel.encode())
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _rows(d, name):
    with open(os.path.join(d, name), newline="") as f:
        return list(csv.DictReader(f))


def _is_split(name):
    return "decode_split" in name or "prefill_tile" in name


def trace_summary(d):
    """Per-kernel stats table and the split kernel's dispatch durations (ns)."""
    stats = _rows(d, "run_kernel_stats.csv")
    disp = _rows(d, "run_kernel_trace.csv")
    split = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in disp if _is_split(r["Kernel_Name"])]
    names = {r["Kernel_Name"] for r in disp if _is_split(r["Kernel_Name"])}
    return stats, split, sorted(names)


def counter_per_dispatch(d, counter):
    """(kernel name, value) per dispatch in dispatch order (values summed over
    the rows rocprofv3 writes for one dispatch)."""
    acc = {}
    order = []
    for r in _rows(d, "run_counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        if key not in acc:
            acc[key] = [r["Kernel_Name"], 0.0]
            order.append(key)
        acc[key][1] += float(r["Counter_Value"])
    return [tuple(acc[k]) for k in sorted(order)]


def split_and_copy(d, counter):
    vals = counter_per_dispatch(d, counter)
    split = [v for n, v in vals if _is_split(n)]
    copies = [v for n, v in vals if "copy" in n.lower() or "elementwise" in n.lower()]
    if len(split) < 2 or not copies:
        raise ValueError(f"{d}: no split dispatches or no calibration copy for {counter}")
    return statistics.median(split[1:]), max(copies)   # drop the warm-up dispatch


def summarize(cfg, trace_dir, fetch_dir, write_dir, bench_json, commands, src_hash=None,
              plain_json=None):
    stats, split_ns, names = trace_summary(trace_dir)
    fetch_kib, fetch_copy = split_and_copy(fetch_dir, "FETCH_SIZE")
    write_kib, write_copy = split_and_copy(write_dir, "WRITE_SIZE")
    ff = COPY_BYTES / 1024.0 / fetch_copy
    wf = COPY_BYTES / 1024.0 / write_copy
    fetch_b = fetch_kib * 1024.0 * ff
    write_b = write_kib * 1024.0 * wf
    with open(bench_json) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    algo = bench["kv_bytes_per_step"]
    k = bench["steps"]
    timed = split_ns[-2 * k:-k] or split_ns  # the timed steps
    b2b = split_ns[-k:]                      # the back-to-back pass the bench brackets with events
    entry = {
        "kernels": names,
        "fetch_bytes": round(fetch_b),
        "write_bytes": round(write_b),
        "fetch_kib_per_dispatch": fetch_kib,
        "write_kib_per_dispatch": write_kib,
        "fetch_factor": round(ff, 4),
        "write_factor": round(wf, 4),
        "algorithmic_bytes": algo,
        "split_avg_us_trace": round(statistics.mean(timed) / 1e3, 3),
        "split_avg_us_trace_b2b": round(statistics.mean(b2b) / 1e3, 3),
        "bench_split_avg_us_events": round(bench["roofline"]["avg_launch_ms"] * 1e3, 3),
        "bench_ms_per_step": bench["ms_per_step"],
    }
    lines = [
        f"# dominant kernel — `{cfg}` workload: kernel trace and HBM counters",
        "",
        f"Workload: {bench['config']['workload']}.",
        f"Timed kernel(s) (the decode split, or the prefill tile kernel): "
        f"{', '.join('`' + n + '`' for n in names)}.",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):",
        "",
        "```",
        *commands,
        "```",
        "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)",
        "",
        "| Kernel | Calls | Average (µs) | Total (ms) |",
        "|---|---|---|---|",
    ]
    for r in stats[:8]:
        nm = r["Name"]
        nm = nm if len(nm) <= 70 else nm[:67] + "..."
        lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} |")
    lines += [
        "",
        f"Split calls include warm-up, the timed steps and the event-timed pass. "
        f"Timed steps ({len(timed)} dispatches): average {entry['split_avg_us_trace']} µs. "
        f"Event-timed pass ({len(b2b)} launches back to back): trace average "
        f"{entry['split_avg_us_trace_b2b']} µs; the bench's HIP-event average over it (elapsed / "
        f"launches, so the gaps between launches count too): "
        f"{entry['bench_split_avg_us_events']} µs. "
        f"Bench line of the trace run: ms_per_step {bench['ms_per_step']}, value "
        f"{bench['value']} GB/s, roofline achieved {bench['roofline']['achieved']} "
        f"{bench['roofline']['unit']}.",
        "",
    ]
    if plain_json:
        # the profiler adds host time to every launch; where a launch is
        # shorter than that, the back-to-back launches starve and the events
        # count the gaps, so the same command is also run without it
        with open(plain_json) as f:
            plain = json.loads(f.read().strip().splitlines()[-1])
        entry["bench_split_avg_us_events_unprofiled"] = round(plain["roofline"]["avg_launch_ms"] * 1e3, 3)
        lines += [
            f"The same bench command without the profiler (`python3 bench.py --config {cfg} "
            f"--steps 50 --warmup 10 --cpu-budget 0`): HIP-event average "
            f"{entry['bench_split_avg_us_events_unprofiled']} µs per split launch, ms_per_step "
            f"{plain['ms_per_step']}, value {plain['value']} GB/s, roofline achieved "
            f"{plain['roofline']['achieved']} {plain['roofline']['unit']}. Under the profiler "
            f"every launch also pays the tracer's host-side cost; where that exceeds the "
            f"kernel's duration the back-to-back launches leave the GPU idle between them "
            f"and the profiled run's event average counts those gaps.",
            "",
        ]
    lines += [
        "## HBM bytes per split dispatch (rocprofv3 --pmc, one counter per run)",
        "",
        "| Counter | KiB per dispatch (median) | 1 GiB copy reads (KiB) | scale | bytes |",
        "|---|---|---|---|---|",
        f"| FETCH_SIZE | {fetch_kib:,.1f} | {fetch_copy:,.1f} | {ff:.3f} | {fetch_b:,.0f} |",
        f"| WRITE_SIZE | {write_kib:,.1f} | {write_copy:,.1f} | {wf:.3f} | {write_b:,.0f} |",
        "",
        f"Algorithmic K/V bytes per launch: {algo:,}; fetched / algorithmic = "
        f"{fetch_b / algo:.4f}.",
        "",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    kernel = "prefill_tile" if any("prefill_tile" in n for n in names) else "decode_split"
    with open(os.path.join(PROFILES, f"{kernel}_{cfg}.md"), "w") as f:
        f.write("\n".join(lines))
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as f:
            data = json.load(f)
    h = src_hash or source_hash()
    if data.get("source_hash") != h:
        data = {"source_hash": h, "configs": {}}
    data["configs"][cfg] = entry
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    return entry


def traffic_bytes(cfg):
    """Scaled FETCH + WRITE bytes of one split launch for workload cfg, or None
    if none were taken or the sources changed since."""
    try:
        with open(TRAFFIC_JSON) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get("configs", {}).get(cfg)
    if not e or data.get("source_hash") != source_hash():
        return None
    return e["fetch_bytes"] + e["write_bytes"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--bench-json", required=True, help="bench.py output of the trace run")
    ap.add_argument("--commands", default="", help="file with the three commands, one per line")
    ap.add_argument("--plain-bench-json", default=None,
                    help="bench.py output of the same command run without the profiler")
    ap.add_argument("--source-hash", default=None,
                    help="source_hash() of the tree the runs were made from (default: this tree)")
    args = ap.parse_args()
    cmds = open(args.commands).read().strip().splitlines() if args.commands else []
    print(json.dumps(summarize(args.config, args.trace, args.fetch, args.write, args.bench_json, cmds,
                               args.source_hash, args.plain_bench_json), indent=1))


if __name__ == "__main__":
    main()
