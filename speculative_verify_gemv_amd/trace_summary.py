"""Kernel durations of the single launches from a rocprofv3 kernel trace.

    python -m speculative_verify_gemv_amd.trace_summary TRACE_CSV ORDER_JSON

TRACE_CSV is the ``*_kernel_trace.csv`` of ``rocprofv3 --kernel-trace
--output-format csv -- python bench.py --singles-pass ORDER_JSON``; ORDER_JSON
lists the workloads in launch order with their untimed and timed call counts
and dispatches per call.  The trace's library dispatches (repacks aside) are
matched to the workloads in that order, and for each workload the timed
calls' kernel durations are summarised: per kernel its median, mean and
minimum, and per call the sum over its dispatches, with the weight bytes per
call divided by that sum against the 8 TB/s HBM peak.  Prints a markdown
table.  Measurement tooling: nothing on the path uses it.
"""
from __future__ import annotations

import csv
import json
import re
import statistics
import sys

HBM_PEAK_GBPS = 8000.0


def short_name(kernel: str) -> str:
    """Kernel name without return type, namespace and argument list."""
    k = re.sub(r"^void ", "", kernel)
    k = k.replace("w4a16::(anonymous namespace)::", "").replace("w4a16::", "")
    return re.sub(r"\(.*", "", k).strip()


def library_dispatches(trace_csv: str) -> list[dict]:
    with open(trace_csv) as f:
        rows = list(csv.DictReader(f))
    rows = [r for r in rows if "w4a16" in r["Kernel_Name"] and "repack" not in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def summarise(trace_csv: str, order_json: str) -> list[dict]:
    rows = library_dispatches(trace_csv)
    with open(order_json) as f:
        order = json.load(f)
    need = sum((o["untimed"] + o["timed"]) * o["dispatches"] for o in order)
    if len(rows) != need:
        raise SystemExit(f"trace holds {len(rows)} library dispatches, the launch order accounts for {need}")
    out, pos = [], 0
    for o in order:
        d = o["dispatches"]
        n = (o["untimed"] + o["timed"]) * d
        timed = rows[pos + o["untimed"] * d: pos + n]
        pos += n
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in timed]
        kernels = []
        for j in range(d):
            ks = dur[j::d]
            r0 = timed[j]
            wgs = int(r0["Grid_Size_X"]) // max(1, int(r0["Workgroup_Size_X"]))
            kernels.append({"kernel": short_name(r0["Kernel_Name"]), "workgroups": wgs,
                            "threads": int(r0["Workgroup_Size_X"]), "median_us": statistics.median(ks),
                            "mean_us": statistics.fmean(ks), "min_us": min(ks)})
        per_call = [sum(dur[i:i + d]) for i in range(0, len(dur), d)]
        med = statistics.median(per_call)
        gbps = o["weight_bytes"] / (med * 1e-6) / 1e9 if o["weight_bytes"] else None
        out.append({"workload": o["workload"], "calls": o["timed"], "kernels": kernels, "call_median_us": med,
                    "call_mean_us": statistics.fmean(per_call), "weight_GBps": gbps,
                    "pct_hbm_peak": None if gbps is None else 100.0 * gbps / HBM_PEAK_GBPS})
    return out


def markdown(res: list[dict]) -> str:
    lines = ["| workload | kernel (workgroups x threads) | median us | mean us | min us | call median us | "
             "weight GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|---|---|"]
    for r in res:
        for i, k in enumerate(r["kernels"]):
            first = i == 0
            lines.append("| {} | {} ({} x {}) | {:.2f} | {:.2f} | {:.2f} | {} | {} | {} |".format(
                r["workload"] if first else "", k["kernel"], k["workgroups"], k["threads"], k["median_us"],
                k["mean_us"], k["min_us"], f"{r['call_median_us']:.2f}" if first else "",
                f"{r['weight_GBps']:.0f}" if first and r["weight_GBps"] else "",
                f"{r['pct_hbm_peak']:.1f}" if first and r["pct_hbm_peak"] else ""))
    return "\n".join(lines)


def main(argv: list[str]) -> None:
    if len(argv) != 3:
        raise SystemExit(__doc__)
    print(markdown(summarise(argv[1], argv[2])))


if __name__ == "__main__":
    main(sys.argv)
