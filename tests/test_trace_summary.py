"""The single-launch trace summary maps a kernel trace back to the launch
order bench.py records (host logic only)."""
import csv
import json

import pytest

from speculative_verify_gemv_amd import trace_summary

pytestmark = pytest.mark.filterwarnings("ignore")

COLS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]
TILE = "void w4a16::(anonymous namespace)::w4a16_tile_kernel<1, 1, false, 1>(w4a16::GemvArgs)"
RUN = "w4a16::(anonymous namespace)::w4a16_run_kernel<1, 1>(w4a16::GemvArgs)"
FINAL = "w4a16::(anonymous namespace)::w4a16_argmax_final(int2 const*, int, int, int*, float*)"
REPACK = "w4a16::(anonymous namespace)::w4a16_repack_kernel(unsigned char const*)"


def write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(COLS)
        for name, t0, dur_ns, wg, threads in rows:
            w.writerow(["KERNEL_DISPATCH", name, t0, t0 + dur_ns, threads, wg * threads])


def test_maps_dispatches_to_workloads_in_order(tmp_path):
    rows, t = [], 1000
    rows.append((REPACK, t, 50_000, 10, 256)); t += 100_000          # ignored
    for i in range(5):                                                # workload a: 2 untimed + 3 timed
        rows.append((TILE, t, 8000 + 1000 * i, 320, 512)); t += 20_000
    for i in range(3):                                                # workload b: 1 untimed + 2 timed, 2 per call
        rows.append((RUN, t, 100_000 + 1000 * i, 243, 1024)); t += 200_000
        rows.append((FINAL, t, 4000, 4, 256)); t += 10_000
    write_trace(tmp_path / "trace.csv", rows)
    order = [{"workload": "a", "untimed": 2, "timed": 3, "dispatches": 1, "weight_bytes": 13_434_880},
             {"workload": "b", "untimed": 1, "timed": 2, "dispatches": 2, "weight_bytes": 635_699_200}]
    (tmp_path / "order.json").write_text(json.dumps(order))
    res = trace_summary.summarise(str(tmp_path / "trace.csv"), str(tmp_path / "order.json"))
    a, b = res
    assert a["kernels"][0]["kernel"] == "w4a16_tile_kernel<1, 1, false, 1>"
    assert a["kernels"][0]["workgroups"] == 320 and a["kernels"][0]["threads"] == 512
    assert a["kernels"][0]["median_us"] == pytest.approx(11.0) and a["kernels"][0]["min_us"] == pytest.approx(10.0)
    assert a["call_median_us"] == pytest.approx(11.0)
    assert a["weight_GBps"] == pytest.approx(13_434_880 / 11e-6 / 1e9)
    assert [k["kernel"] for k in b["kernels"]] == ["w4a16_run_kernel<1, 1>", "w4a16_argmax_final"]
    assert b["kernels"][0]["median_us"] == pytest.approx(101.5)
    assert b["call_median_us"] == pytest.approx(105.5)
    table = trace_summary.markdown(res)
    assert table.count("\n") == 2 + 2 and "w4a16_argmax_final" in table


def test_count_mismatch_is_an_error(tmp_path):
    write_trace(tmp_path / "trace.csv", [(TILE, 0, 1000, 1, 64)])
    (tmp_path / "order.json").write_text(json.dumps(
        [{"workload": "a", "untimed": 1, "timed": 1, "dispatches": 1, "weight_bytes": 0}]))
    with pytest.raises(SystemExit):
        trace_summary.summarise(str(tmp_path / "trace.csv"), str(tmp_path / "order.json"))


def test_runs_group_by_kernel_and_shape(tmp_path):
    rows, t = [], 0
    rows.append((REPACK, t, 40_000, 4620, 256)); t += 50_000
    rows.append((REPACK, t, 10_000, 3300, 256)); t += 50_000
    for _ in range(3):
        rows.append((RUN, t, 100_000, 243, 1024)); t += 200_000
        rows.append((FINAL, t, 5000, 4, 256)); t += 10_000
    for i in range(2):
        rows.append((TILE, t, 8000, 320, 512)); t += 20_000
    rows.append((RUN, t, 90_000, 243, 1024))
    write_trace(tmp_path / "trace.csv", rows)
    runs = trace_summary._runs(str(tmp_path / "trace.csv"))
    got = [(r["sig"][0], r["sig"][1], len(r["d"])) for r in runs]
    assert got == [("w4a16_run_kernel<1, 1>", 243, 4), ("w4a16_repack_kernel", 0, 2),
                   ("w4a16_tile_kernel<1, 1, false, 1>", 320, 2), ("w4a16_argmax_final", 4, 3)]
    assert sorted(runs[0]["d"]) == [90.0, 100.0, 100.0, 100.0]
    assert trace_summary.runs_markdown(str(tmp_path / "trace.csv")).count("\n") == 2 + 3


def test_traffic_is_calibrated_by_the_copy(tmp_path):
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    disp = [(1, REPACK, 2560, 256), (2, "__amd_rocclr_copyBuffer", 1 << 20, 256), (3, RUN, 243 * 1024, 1024),
            (4, FINAL, 4 * 256, 256), (5, TILE, 320 * 512, 512)]
    fetch = {1: 10.0, 2: 524288.0, 3: 1000.0, 4: 2.0, 5: 300.0}      # the copy: 0.5 GiB for 1 GiB read
    write = {1: 5.0, 2: 1048576.0, 3: 64.0, 4: 1.0, 5: 16.0}
    for name, vals, counter in (("f.csv", fetch, "FETCH_SIZE"), ("w.csv", write, "WRITE_SIZE")):
        with open(tmp_path / name, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(cols)
            for d, k, g, wg in disp:
                w.writerow([d, k, g, wg, counter, vals[d]])
    text, step = trace_summary.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "ab" * 32)
    assert step == 2 * 1000 * 1024 + 64 * 1024        # fetched counts twice, written once
    assert f"traffic_bytes_per_launch: {step}" in text and "kernel_source_sha256: " + "ab" * 32 in text
    assert "w4a16_tile_kernel<1, 1, false, 1>" in text and "repack" not in text


def test_counters_map_the_launch_order(tmp_path):
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    disp = [(1, REPACK), (2, TILE), (3, RUN), (4, FINAL)]
    with open(tmp_path / "sq.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for d, k in disp:
            w.writerow([d, k, 64, 64, "SQ_INSTS_VALU", 1000.0 * d])
            w.writerow([d, k, 64, 64, "SQ_INSTS_MFMA", 10.0 * d])
    with open(tmp_path / "fetch.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for d, k in disp:
            w.writerow([d, k, 64, 64, "FETCH_SIZE", 4.0 * d])
    with open(tmp_path / "calib.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerow([1, "__amd_rocclr_copyBuffer", 64, 64, "FETCH_SIZE", 524288.0])
    order = [{"workload": "a", "untimed": 0, "timed": 1, "dispatches": 1, "weight_bytes": 8192},
             {"workload": "b", "untimed": 0, "timed": 1, "dispatches": 2, "weight_bytes": 16384}]
    (tmp_path / "order.json").write_text(json.dumps(order))
    table = trace_summary.counters(str(tmp_path / "order.json"), str(tmp_path / "calib.csv"),
                                   [str(tmp_path / "sq.csv"), str(tmp_path / "fetch.csv")])
    lines = table.splitlines()
    assert lines[0].startswith("| workload | kernel | FETCH_SIZE | SQ_INSTS_MFMA | SQ_INSTS_VALU | VALU / KB |")
    # a: dispatch 2 (2000 VALU over 8 KB); b: dispatches 3 + 4 (7000 VALU over 16 KB)
    assert "| a | w4a16_tile_kernel<1, 1, false, 1> | 8 | 20 | 2e+03 | 250.0 | 2.000 |" == lines[2]
    assert "| b | w4a16_run_kernel<1, 1> | 28 | 70 | 7e+03 | 437.5 | 3.500 |" == lines[3]
