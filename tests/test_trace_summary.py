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
