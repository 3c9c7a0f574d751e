"""Summaries of rocprofv3 output for bench.py's runs (markdown tables).

    python -m speculative_verify_gemv_amd.trace_summary TRACE_CSV ORDER_JSON
    python -m speculative_verify_gemv_amd.trace_summary runs TRACE_CSV
    python -m speculative_verify_gemv_amd.trace_summary traffic FETCH_CSV WRITE_CSV
    python -m speculative_verify_gemv_amd.trace_summary counters ORDER_JSON CALIB_FETCH_CSV CSV [CSV ...]

Single launches: TRACE_CSV is the ``*_kernel_trace.csv`` of ``rocprofv3
--kernel-trace --output-format csv -- python bench.py --singles-pass
ORDER_JSON``; ORDER_JSON lists the workloads in launch order with their
untimed and timed call counts and dispatches per call.  The trace's library
dispatches (repacks aside) are matched to the workloads in that order, and
for each workload the timed calls' kernel durations are summarised: per
kernel its median, mean and minimum, and per call the sum over its
dispatches, with the weight bytes per call divided by that sum against the
8 TB/s HBM peak.

runs: a whole kernel trace (e.g. of ``python bench.py``) grouped by kernel
and launch shape (the load-time repacks on one line), in order of total
time; per group the call count, the average, median and minimum kernel
durations and the total.

traffic: two counter-collection CSVs of ``bench.py --pmc-pass``, one with
FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch).  The pass first copies
1 GiB with torch's copy kernel; what the counters read for that copy gives
the factors from counter units to bytes, applied to every library dispatch
after it.  Prints the calibrated bytes per dispatch and, for the step's
grouped launch (the first library dispatch after the copy), the
``traffic_bytes_per_launch`` and ``kernel_source_sha256`` lines bench.py
reads back.

counters: counter-collection CSVs of a pass that wrote a launch order
(``bench.py --variants-pass ORDER_JSON``), each workload's dispatches summed
per counter (all its dispatches: the head kernel with its argmax reduction);
SQ_INSTS_VALU is also given per KB of weight bytes and FETCH_SIZE as a ratio
to the weight bytes, calibrated by the copy in CALIB_FETCH_CSV (the
FETCH_SIZE pass of ``bench.py --pmc-pass``).

Measurement tooling: nothing on the path uses it.
"""
from __future__ import annotations

import csv
import json
import os
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


def _runs(trace_csv: str) -> list[dict]:
    """Library dispatches grouped by (kernel, workgroups, threads) over the
    whole trace, in order of total time."""
    with open(trace_csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    groups: dict = {}
    for r in rows:
        if "w4a16" not in r["Kernel_Name"]:
            continue
        name = short_name(r["Kernel_Name"])
        wg = max(1, int(r["Workgroup_Size_X"]))
        sig = (name, int(r["Grid_Size_X"]) // wg, wg)
        if "repack" in name:  # load-time repacks: one line for all shapes
            sig = (name, 0, wg)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        groups.setdefault(sig, {"sig": sig, "d": []})["d"].append(dur)
    return sorted(groups.values(), key=lambda g: -sum(g["d"]))


def runs_markdown(trace_csv: str) -> str:
    lines = ["| kernel | workgroups x threads | calls | avg us | median us | min us | total ms |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for r in _runs(trace_csv):
        name, wgs, threads = r["sig"]
        d = r["d"]
        shape = f"(all) x {threads}" if wgs == 0 else f"{wgs} x {threads}"
        lines.append(f"| {name} | {shape} | {len(d)} | {statistics.fmean(d):.2f} | {statistics.median(d):.2f} | "
                     f"{min(d):.2f} | {sum(d) / 1000:.2f} |")
    return "\n".join(lines)


COPY_BYTES = 1 << 30


def _counters(path: str, counter: str) -> list[tuple[str, int, int, float]]:
    """(kernel name, workgroups, threads, value) per dispatch, in dispatch order."""
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])), int(r["Workgroup_Size"]),
             float(r["Counter_Value"])) for r in rows]


def traffic(fetch_csv: str, write_csv: str, source_hash: str | None = None) -> tuple[str, int]:
    fetch, write = _counters(fetch_csv, "FETCH_SIZE"), _counters(write_csv, "WRITE_SIZE")
    if len(fetch) != len(write) or any(a[0] != b[0] for a, b in zip(fetch, write)):
        raise SystemExit("the two passes dispatched different kernels")
    copy = [i for i, r in enumerate(fetch) if "w4a16" not in r[0] and "copy" in r[0].lower()]
    if not copy:
        raise SystemExit("no copy kernel before the library dispatches")
    c = copy[0]
    f_factor = COPY_BYTES / (fetch[c][3] * 1024.0)
    w_factor = COPY_BYTES / (write[c][3] * 1024.0)
    lines = [f"Calibration: the 1 GiB copy reads FETCH_SIZE {fetch[c][3]:,.2f} KiB and WRITE_SIZE "
             f"{write[c][3]:,.2f} KiB, so fetched bytes = {f_factor:.5f} x FETCH_SIZE x 1024 and written bytes = "
             f"{w_factor:.5f} x WRITE_SIZE x 1024.", "",
             "| dispatch | kernel | workgroups x threads | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched B | written B |",
             "|---:|---|---|---:|---:|---:|---:|"]
    step = None
    for i in range(c + 1, len(fetch)):
        name, wgs, threads, fv = fetch[i]
        if "w4a16" not in name or "repack" in name:
            continue
        wv = write[i][3]
        fb, wb = round(fv * 1024 * f_factor), round(wv * 1024 * w_factor)
        if step is None:
            step = fb + wb
        lines.append(f"| {i} | {short_name(name)} | {wgs} x {threads} | {fv:,.2f} | {wv:,.2f} | {fb:,} | {wb:,} |")
    if step is None:
        raise SystemExit("no library dispatch after the copy")
    lines += ["", f"traffic_bytes_per_launch: {step}"]
    if source_hash:
        lines.append(f"kernel_source_sha256: {source_hash}")
    return "\n".join(lines), step


def _by_dispatch(path: str) -> list[tuple[str, dict]]:
    """(kernel name, {counter: value}) per library dispatch (repacks aside), in order."""
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if "w4a16" in r["Kernel_Name"] and "repack" not in r["Kernel_Name"]]
    d: dict = {}
    for r in rows:
        k = int(r["Dispatch_Id"])
        d.setdefault(k, (r["Kernel_Name"], {}))[1][r["Counter_Name"]] = float(r["Counter_Value"])
    return [d[k] for k in sorted(d)]


def counters(order_json: str, calib_fetch_csv: str, csvs: list[str]) -> str:
    with open(order_json) as f:
        order = json.load(f)
    fetch = _counters(calib_fetch_csv, "FETCH_SIZE")
    copy = [r for r in fetch if "w4a16" not in r[0] and "copy" in r[0].lower()]
    f_factor = COPY_BYTES / (copy[0][3] * 1024.0) if copy else None
    merged: list[tuple[str, dict]] = []
    for path in csvs:
        rows = _by_dispatch(path)
        if not merged:
            merged = [(k, dict(v)) for k, v in rows]
        else:
            if len(rows) != len(merged) or any(a[0] != b[0] for a, b in zip(rows, merged)):
                raise SystemExit(f"{path} dispatched different kernels")
            for (_, acc), (_, v) in zip(merged, rows):
                acc.update(v)
    need = sum((o["untimed"] + o["timed"]) * o["dispatches"] for o in order)
    if len(merged) != need:
        raise SystemExit(f"{len(merged)} library dispatches, the launch order accounts for {need}")
    names = sorted({c for _, v in merged for c in v})
    head = ["workload", "kernel"] + names + (["VALU / KB"] if "SQ_INSTS_VALU" in names else [])
    if "FETCH_SIZE" in names and f_factor:
        head.append("fetch / weight bytes")
    lines = ["| " + " | ".join(head) + " |", "|" + "---|" * 2 + "---:|" * (len(head) - 2)]
    pos = 0
    for o in order:
        n = (o["untimed"] + o["timed"]) * o["dispatches"]
        part = merged[pos + o["untimed"] * o["dispatches"]: pos + n]
        pos += n
        tot = {c: sum(v.get(c, 0.0) for _, v in part) for c in names}
        cells = [o["workload"], short_name(part[0][0])] + [f"{tot[c]:.3g}" for c in names]
        if "SQ_INSTS_VALU" in names:
            cells.append(f"{tot['SQ_INSTS_VALU'] / (o['weight_bytes'] / 1024.0):.1f}")
        if "FETCH_SIZE" in names and f_factor:
            cells.append(f"{tot['FETCH_SIZE'] * 1024 * f_factor / o['weight_bytes']:.3f}")
        lines.append("| " + " | ".join(cells) + " |")
    return "\n".join(lines)


def main(argv: list[str]) -> None:
    if len(argv) == 3 and argv[1] == "runs":
        print(runs_markdown(argv[2]))
    elif len(argv) == 4 and argv[1] == "traffic":
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        from speculative_verify_gemv_amd.metrics import kernel_source_hash
        print(traffic(argv[2], argv[3], kernel_source_hash())[0])
    elif len(argv) >= 5 and argv[1] == "counters":
        print(counters(argv[2], argv[3], argv[4:]))
    elif len(argv) == 3:
        print(markdown(summarise(argv[1], argv[2])))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
