"""Benchmark: the decode weight pass of a 27B-class model on one MI355X.

One step is one verify cycle's weight read: 64 layers x {qkv, o, gate_up,
down} W4A16 projections and the 248,320-row lm_head with per-row argmax, at
T = 4 (1 + 3 drafts), each matrix with its own seeded weights and
activations, all in one grouped launch (followed by the argmax reduction, a
launch of T workgroups).  Weights are repacked once at load into the tiled
layout (same codes and scales, one contiguous 1 KB block per 16 rows x 128
columns) and stay resident in HBM; nothing is cached between steps (11.6 GB
per step, far beyond the 256 MB Infinity Cache).

Reported (one JSON line): weight GB/s of the whole step (value), decode
cycles/s, the grouped kernel's achieved bandwidth against the 8 TB/s HBM
peak (roofline, timed with HIP events on the launch stream), the same step
as two launches (body pass, then the lm_head) and as 257 separate launches
replayed from a captured HIP graph, the body pass alone at T = 1, 4, 8 and
16 in both layouts (tiled and the pages' row-major one), single launches of
each workload shape (the small matrix, every projection at T = 1, 4, 8, the
lm_head with argmax, the draft head), the dot-product variant against the
matrix-core one on the same single launches, the achievable streaming-read
rate, the verify epilogue, and the CPU oracle's rate on a bounded sample
(cpu_baseline), with the parity of the last timed step against the oracle
(every output of layer 0 and every lm_head score, the argmax ids), checked
after the timing.

--pmc-pass runs one untimed step after a 1 GiB device copy (the calibration
kernel for rocprofv3 FETCH_SIZE/WRITE_SIZE), then one body pass alone at
each of T = 1, 4, 8, 16;
--variants-pass [ORDER_JSON] one untimed launch per shape, T and variant
(writing their launch order when given); --singles-pass ORDER_JSON the
single launches alone, then the streaming-read floor of each size, writing
their launch order (trace_summary maps kernel traces and counter passes
back to either order).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from speculative_verify_gemv_amd import metrics  # noqa: E402

METRIC = "weight GB/s and % of HBM peak at T=1/4/8 (27B-class shapes); decode cycles/s"
PEAK_GBPS = 8000.0
WORKLOAD = "decode_weight_pass_64x(qkv,o,gate_up,down)+lm_head_T4"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_body_pass_T4.md")
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--T", type=int, default=4)
    ap.add_argument("--layers", type=int, default=synth.LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-t", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-singles", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true", help="one untimed pass for counter collection")
    ap.add_argument("--variants-pass", nargs="?", const="", default=None, metavar="ORDER_JSON",
                    help="one untimed launch per shape, T and kernel variant (dot / matrix core), for counters; "
                         "writes the launch order to ORDER_JSON when given")
    ap.add_argument("--singles-pass", metavar="ORDER_JSON",
                    help="run only the single launches and write their launch order here (for a kernel trace)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a, torch):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


def measured_traffic():
    """HBM bytes per body-pass launch from the committed counter summary, or
    None when it is absent or was taken on a different kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    b = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not h or not b or h.group(1) != metrics.kernel_source_hash():
        return None
    return int(b.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the W4A16 pass is measured on a single "
              "MI355X and is not sharded here.", file=sys.stderr)
        sys.exit(2)
    import torch
    import speculative_verify_gemv_amd as w4a16

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w4a16.load_library()
    T = args.T
    L = args.layers
    t0 = time.time()

    # ---- resident weights: 64 layers x 4 projections + lm_head (seeded) ----
    weights = []  # (name, layer, packed_dev, scales_dev, tiled)
    for layer in range(L):
        for proj in synth.PROJ_ORDER:
            N, K = synth.PROJECTIONS[proj]
            p, s = synth.weight(synth.tid_layer(layer, proj), N, K)
            pd, sd = to_dev(p, torch), to_dev(s, torch)
            weights.append((proj, layer, pd, sd, w4a16.repack_tiled(pd, sd)))
    hn, hk = synth.LM_HEAD
    hp, hs = synth.weight(synth.TID_LM_HEAD, hn, hk)
    head_p, head_s = to_dev(hp, torch), to_dev(hs, torch)
    head_tw = w4a16.repack_tiled(head_p, head_s)
    del hp, hs
    torch.cuda.synchronize()
    log(f"weights resident (row-major and tiled) after {time.time() - t0:.1f} s")

    body_bytes = sum(metrics.weight_bytes(*synth.PROJECTIONS[w[0]]) for w in weights)
    head_bytes = metrics.weight_bytes(hn, hk)

    def make_pass(Tp, tiled=True):
        probs = []
        for proj, layer, pd, sd, tw in weights:
            N, K = synth.PROJECTIONS[proj]
            x = to_dev(synth.activations(synth.tid_layer(layer, proj), Tp, K), torch)
            y = torch.empty((Tp, N), dtype=torch.float32, device="cuda")
            probs.append((tw, None, x, y) if tiled else (pd, sd, x, y))
        return w4a16.Batch(probs, Tp), probs

    batch, probs = make_pass(T)
    head_x = to_dev(synth.activations(synth.TID_LM_HEAD, T, hk), torch)
    head_y = torch.empty((T, hn), dtype=torch.float32, device="cuda")
    head_ws = torch.empty(w4a16.workspace_bytes(hn, T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    head_id = torch.empty(T, dtype=torch.int32, device="cuda")
    head_val = torch.empty(T, dtype=torch.float32, device="cuda")

    def head(s):
        w4a16.head_gather_tiled(head_tw, head_x, scores=True, argmax=True, out=head_y, workspace=head_ws, stream=s)

    # the step: the 256 projections and the lm_head with its argmax in one
    # grouped launch (then the argmax reduction, a small launch of T workgroups)
    step = w4a16.Batch(probs + [(head_tw, None, head_x, head_y, head_id, head_val, head_ws)], T)

    if args.variants_pass is not None:
        order = variants_pass(torch, w4a16, weights, head_p, head_s, stream)
        if args.variants_pass:
            with open(args.variants_pass, "w") as f:
                json.dump(order, f, indent=1)
        return

    if args.singles_pass:
        single_launches(torch, w4a16, weights, head_p, head_s, head_tw, stream)
        read_floors(torch, w4a16, stream)
        with open(args.singles_pass, "w") as f:
            json.dump(LAUNCH_ORDER, f, indent=1)
        log(f"singles pass done: launch order of {len(LAUNCH_ORDER)} workloads in {args.singles_pass}")
        return

    if args.pmc_pass:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)  # calibration: reads and writes exactly 1 GiB
        step.run(stream)
        for Tp in (1, 4, 8, 16):  # the body pass alone at each verify width
            b, _ = (batch, probs) if Tp == T else make_pass(Tp)
            b.run(stream)
            torch.cuda.synchronize()
            del b
        torch.cuda.synchronize()
        log(f"pmc pass done: copy {COPY_BYTES} B, step {body_bytes + head_bytes} B at T = {T}, "
            f"body pass at T = 1, 4, 8, 16")
        return

    def time_step(st, steps, warmup):
        """Whole-loop and per-launch times of `steps` grouped launches (each
        followed by its argmax reduction), after `warmup` untimed ones."""
        for _ in range(warmup):
            st.run(stream)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(steps):
            ev[i][0].record(stream)
            st.run(stream)
            ev[i][1].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) for a, b in ev]
        return start.elapsed_time(end) / steps, per

    step_bytes = body_bytes + head_bytes
    ms_step, launch_ms = time_step(step, args.steps, args.warmup)
    K_steps = args.steps
    # the last timed step's outputs, kept for the parity check of the CPU
    # baseline leg (layer 0's four projections and the lm_head)
    torch.cuda.synchronize()
    step_out = {"layer0": [(proj, y.cpu().numpy()) for (proj, layer, *_), (*_, y) in zip(weights, probs) if layer == 0],
                "head_y": head_y.cpu().numpy(), "head_id": head_id.cpu().numpy()}
    launch_ms_avg = float(np.mean(launch_ms))
    value = metrics.gbps(step_bytes, ms_step)
    achieved = metrics.gbps(step_bytes, launch_ms_avg)
    log(f"step {ms_step:.4f} ms, grouped launch + argmax reduction {launch_ms_avg:.4f} ms "
        f"(median {np.median(launch_ms):.4f}, min {min(launch_ms):.4f}), {value:.0f} GB/s per step, "
        f"kernel {achieved:.0f} GB/s")

    # the same step (body + lm_head with argmax, one grouped launch) at the
    # other verify widths: T = 1 (plain decode) and T = 8
    per_t_step = {f"T{T}": step_summary(step_bytes, ms_step, launch_ms)}
    for Tp in (1, 8):
        if Tp == T:
            continue
        b_probs = make_pass(Tp)[1]
        hxp = to_dev(synth.activations(synth.TID_LM_HEAD, Tp, hk), torch)
        hyp = torch.empty((Tp, hn), dtype=torch.float32, device="cuda")
        hwp = torch.empty(w4a16.workspace_bytes(hn, Tp), dtype=torch.uint8, device="cuda")
        hip_ = torch.empty(Tp, dtype=torch.int32, device="cuda")
        hvp = torch.empty(Tp, dtype=torch.float32, device="cuda")
        st = w4a16.Batch(b_probs + [(head_tw, None, hxp, hyp, hip_, hvp, hwp)], Tp)
        ms_p, per_p = time_step(st, args.steps, args.warmup)
        per_t_step[f"T{Tp}"] = step_summary(step_bytes, ms_p, per_p)
        log(f"step T={Tp}: {ms_p:.4f} ms ({per_t_step[f'T{Tp}']['cycles_per_s']} cycles/s), launch "
            f"{np.mean(per_p):.4f} ms, {per_t_step[f'T{Tp}']['roofline']['frac']:.4f} of 8 TB/s")
        del st, b_probs
    per_t_step = {k: per_t_step[k] for k in sorted(per_t_step, key=lambda k: int(k[1:]))}

    # the same step as two launches (body pass, then the lm_head with argmax)
    for _ in range(5):
        batch.run(stream)
        head(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K_steps):
        batch.run(stream)
        head(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_two = e0.elapsed_time(e1) / K_steps
    log(f"step as body pass + separate lm_head launch: {ms_two:.4f} ms, {metrics.gbps(step_bytes, ms_two):.0f} GB/s")

    # ---- body pass at T = 1, 4, 8, 16 (same weights, grouped launch), both layouts ----
    per_t, per_t_rm = {}, {}
    if not args.no_per_t:
        for tiled, table in ((True, per_t), (False, per_t_rm)):
            for Tp in (1, 4, 8, 16):
                b, _ = (batch, probs) if (Tp == T and tiled) else make_pass(Tp, tiled)
                for _ in range(20):  # ~40 ms of work: past the clock ramp after the host-side set-up
                    b.run(stream)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 20
                e0.record(stream)
                for _ in range(reps):
                    b.run(stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                g = metrics.gbps(body_bytes, ms)
                table[f"T{Tp}"] = {"body_ms": round(ms, 4), "weight_GBps": round(g, 1),
                                   "pct_hbm_peak": round(100 * g / PEAK_GBPS, 2)}
                log(f"body pass {'tiled' if tiled else 'row-major'} T={Tp}: {ms:.4f} ms, {g:.0f} GB/s "
                    f"({100 * g / PEAK_GBPS:.1f}% of 8 TB/s)")
                del b

    # ---- single launches of each workload shape (configs of the task's workload list) ----
    singles = None
    if not args.no_singles:
        singles = single_launches(torch, w4a16, weights, head_p, head_s, head_tw, stream)

    # ---- the dot-product variant against the matrix-core one (row-major weights) ----
    variants = None
    if not args.no_variants:
        variants = variant_launches(torch, w4a16, weights, head_p, head_s, stream)

    # ---- achievable streaming-read ceiling (context for the 8 TB/s peak) ----
    ceiling = read_ceiling(torch, w4a16, stream)
    log(f"streaming-read ceiling: {ceiling['GBps']:.0f} GB/s ({ceiling['bytes'] >> 30} GiB, "
        f"{ceiling['workgroups']} workgroups)")

    # ---- verify epilogue on the head's scores: top-32 per row, greedy acceptance ----
    epilogue = verify_epilogue(torch, w4a16, head_y, T, stream)
    log(f"verify epilogue at T={T}: top-32 of {hn} scores {epilogue['topk32_us']:.1f} us, "
        f"greedy acceptance {epilogue['greedy_us']:.1f} us, draft-head id list {epilogue['draft_union_us']:.1f} us")

    # ---- the same step as 257 separate launches, replayed from a HIP graph ----
    graph_pass = plain_pass = None
    if not args.no_graph:
        graph_pass = graph_step(torch, w4a16, probs, head, reps=10)
        g = metrics.gbps(step_bytes, graph_pass["ms_per_step"])
        graph_pass["weight_GBps"] = round(g, 1)
        log(f"257-launch graph step: {graph_pass['ms_per_step']:.4f} ms, {g:.0f} GB/s")
        plain_pass = plain_launch_step(torch, w4a16, probs, head, stream, reps=10)
        g = metrics.gbps(step_bytes, plain_pass["ms_per_step"])
        plain_pass["weight_GBps"] = round(g, 1)
        log(f"257 plain stream launches: {plain_pass['ms_per_step']:.4f} ms, {g:.0f} GB/s")

    # ---- CPU baseline: the oracle on a bounded sample of the same pass ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(T, args.cpu_seconds, step_out)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x bf16 activations (exact fp16 products), fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {
            "workload": WORKLOAD,
            "T": T,
            "layers": L,
            "projections": {k: list(v) for k, v in synth.PROJECTIONS.items()},
            "lm_head": [hn, hk],
            "group": 128,
            "weight_bytes_per_step": step_bytes,
            "layout": "tiled (load-time repack of the row-major codes and scales)",
        },
        "cycles_per_s": round(1000.0 / ms_step, 2),
        "pct_hbm_peak": round(100 * value / PEAK_GBPS, 2),
        "per_T_step": per_t_step,
        "per_T_body_pass": per_t,
        "per_T_body_pass_row_major": per_t_rm,
        "step_two_launches": {"ms_per_step": round(ms_two, 4),
                              "weight_GBps": round(metrics.gbps(step_bytes, ms_two), 1)},
        "graph_257_launches": graph_pass,
        "plain_257_launches": plain_pass,
        "verify_epilogue": epilogue,
        "single_launches": singles,
        "variants_dot_vs_matrix_core": variants,
        "read_ceiling": ceiling,
        "device": device_info(torch),
        "roofline": {
            "kernel": "grouped launch of the step (64 x 4 projections + lm_head with argmax, tiled layout); "
                      "the launch time includes the argmax reduction launched after it",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": step_bytes,
            "avg_launch_ms": round(launch_ms_avg, 4),
            "median_launch_ms": round(float(np.median(launch_ms)), 4),
            "min_launch_ms": round(float(min(launch_ms)), 4),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def step_summary(step_bytes, ms_step, launch_ms):
    """cycles/s and the roofline of one verify width's step: the launch
    (grouped kernel + argmax reduction) timed with HIP events on its stream."""
    avg = float(np.mean(launch_ms))
    g = metrics.gbps(step_bytes, avg)
    return {"ms_per_step": round(ms_step, 4), "cycles_per_s": round(1000.0 / ms_step, 2),
            "weight_GBps": round(metrics.gbps(step_bytes, ms_step), 1),
            "roofline": {"bound": "hbm", "achieved": round(g, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                         "frac": round(g / PEAK_GBPS, 4), "avg_launch_ms": round(avg, 4),
                         "median_launch_ms": round(float(np.median(launch_ms)), 4),
                         "min_launch_ms": round(float(min(launch_ms)), 4)}}


def device_info(torch):
    """Name, architecture and size of the GPU the figures were measured on
    (box-to-box spread of the same library is several percent)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1)}
    for attr in ("clock_rate", "memory_clock_rate", "L2_cache_size"):
        if getattr(p, attr, None) is not None:
            info[attr] = getattr(p, attr)
    return info


# (workload, untimed calls, timed calls, dispatches per call, weight bytes)
# of every time_rotating call in order: maps a kernel trace back to them
LAUNCH_ORDER = []


def time_rotating(torch, fns, stream, rounds=4, tag=None, dispatches=1, nbytes=0):
    """Average µs per call of fns called round-robin (distinct weight copies,
    so that the 256 MB Infinity Cache cannot serve a repeat), after one
    untimed round per copy and enough calls to leave the clock ramp."""
    n = len(fns)
    warm = max(3 * n, 30)
    LAUNCH_ORDER.append({"workload": tag, "untimed": warm, "timed": max(rounds * n, 40), "dispatches": dispatches,
                         "weight_bytes": nbytes})
    for i in range(warm):
        fns[i % n]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(rounds * n, 40)
    e0.record(stream)
    for i in range(reps):
        fns[i % n]()
    e1.record(stream)
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / reps


def single_launches(torch, w4a16, weights, head_p, head_s, head_tw, stream):
    """One launch per call, back to back on one stream, for each single-matmul
    workload: the 1024 x 1024 matrix (T = 1), each 27B-class projection at
    T = 1, 4, 8 (tiled, copies from all 64 layers rotated), the lm_head at
    T = 1 and 4 with argmax, and the 32,768-row draft head at T = 1, gathered
    from the row-major head (and, for comparison, from the tiled one) and
    repacked once as its own matrix."""
    out = {}
    # small matrix: too small for any cache effect to matter; its figure is latency
    p, s = synth.weight(synth.TID_SMALL, *synth.SMALL)
    tw = w4a16.repack_tiled(to_dev(p, torch), to_dev(s, torch))
    x = to_dev(synth.activations(synth.TID_SMALL, 1, synth.SMALL[1]), torch)
    y = torch.empty((1, synth.SMALL[0]), dtype=torch.float32, device="cuda")
    us = time_rotating(torch, [lambda: w4a16.matmul_tiled(tw, x, out=y, stream=stream)], stream,
                       tag="small_1024x1024_T1", nbytes=metrics.weight_bytes(*synth.SMALL))
    out["small_1024x1024_T1"] = {"us": round(us, 2),
                                 "weight_GBps": round(metrics.gbps(metrics.weight_bytes(*synth.SMALL), us / 1000), 1)}
    for proj in synth.PROJ_ORDER:
        N, K = synth.PROJECTIONS[proj]
        tws = [w[4] for w in weights if w[0] == proj]
        wb = metrics.weight_bytes(N, K)
        for T in (1, 4, 8):
            x = to_dev(synth.activations(synth.tid_layer(0, proj), T, K), torch)
            y = torch.empty((T, N), dtype=torch.float32, device="cuda")
            fns = [lambda tw=tw: w4a16.matmul_tiled(tw, x, out=y, stream=stream) for tw in tws]
            us = time_rotating(torch, fns, stream, tag=f"{proj}_T{T}", nbytes=wb)
            out[f"{proj}_T{T}"] = {"us": round(us, 2), "weight_GBps": round(metrics.gbps(wb, us / 1000), 1)}
    hn, hk = synth.LM_HEAD
    head_tw2 = w4a16.repack_tiled(head_p, head_s)  # a second copy: 1.3 GB rotated
    for T in (1, 4):
        x = to_dev(synth.activations(synth.TID_LM_HEAD + 1, T, hk), torch)
        y = torch.empty((T, hn), dtype=torch.float32, device="cuda")
        ws = torch.empty(w4a16.workspace_bytes(hn, T), dtype=torch.uint8, device="cuda")
        fns = [lambda t=t: w4a16.head_gather_tiled(t, x, scores=True, argmax=True, out=y, workspace=ws, stream=stream)
               for t in (head_tw, head_tw2)]
        us = time_rotating(torch, fns, stream, tag=f"lm_head_argmax_T{T}", dispatches=2,
                           nbytes=metrics.weight_bytes(hn, hk))
        out[f"lm_head_argmax_T{T}"] = {"us": round(us, 2),
                                       "weight_GBps": round(metrics.gbps(metrics.weight_bytes(hn, hk), us / 1000), 1)}
    ids = [to_dev(synth.distinct_ids(synth.RID_DRAFT + i, synth.DRAFT_IDS, hn), torch) for i in range(8)]
    x = to_dev(synth.activations(synth.TID_LM_HEAD + 2, 1, hk), torch)
    y = torch.empty((1, synth.DRAFT_IDS), dtype=torch.float32, device="cuda")
    ws = torch.empty(w4a16.workspace_bytes(synth.DRAFT_IDS, 1), dtype=torch.uint8, device="cuda")
    # gathered from the row-major head (a row's consecutive groups share
    # 128-byte lines), eight id sets rotated; and from the tiled head
    fns = [lambda r=r: w4a16.head_gather(head_p, head_s, x, row_ids=r, scores=True, argmax=True, out=y, workspace=ws,
                                         stream=stream) for r in ids]
    us = time_rotating(torch, fns, stream, tag="draft_head_32768_argmax_T1", dispatches=2,
                       nbytes=metrics.weight_bytes(synth.DRAFT_IDS, hk))
    out["draft_head_32768_argmax_T1"] = {"us": round(us, 2), "weight_GBps": round(
        metrics.gbps(metrics.weight_bytes(synth.DRAFT_IDS, hk), us / 1000), 1), "layout": "row-major head"}
    fns = [lambda t=t, r=r: w4a16.head_gather_tiled(t, x, row_ids=r, scores=True, argmax=True, out=y, workspace=ws,
                                                    stream=stream) for t in (head_tw, head_tw2) for r in ids[:4]]
    us = time_rotating(torch, fns, stream, tag="draft_head_32768_argmax_T1_tiled_head", dispatches=2,
                       nbytes=metrics.weight_bytes(synth.DRAFT_IDS, hk))
    out["draft_head_32768_argmax_T1_tiled_head"] = {"us": round(us, 2), "weight_GBps": round(
        metrics.gbps(metrics.weight_bytes(synth.DRAFT_IDS, hk), us / 1000), 1), "layout": "tiled head"}
    # the same draft head repacked once into its own tiled matrix (ascending
    # ids, so the argmax position indexes them); 12 copies rotated (1 GB)
    sid = [torch.sort(r)[0] for r in ids[:1]]
    compact = [w4a16.repack_tiled_rows(head_p, head_s, sid[0]) for _ in range(12)]
    fns = [lambda t=t: w4a16.head_gather_tiled(t, x, scores=True, argmax=True, out=y, workspace=ws, stream=stream)
           for t in compact]
    us = time_rotating(torch, fns, stream, tag="draft_head_compact_32768_argmax_T1", dispatches=2,
                       nbytes=metrics.weight_bytes(synth.DRAFT_IDS, hk))
    out["draft_head_compact_32768_argmax_T1"] = {"us": round(us, 2), "weight_GBps": round(
        metrics.gbps(metrics.weight_bytes(synth.DRAFT_IDS, hk), us / 1000), 1)}
    del head_tw2, compact
    for k, v in out.items():
        log(f"single launch {k}: {v['us']:.1f} us, {v['weight_GBps']:.0f} GB/s")
    return out


VARIANT_SHAPES = ("qkv", "o", "gate_up", "down")


def variant_launches(torch, w4a16, weights, head_p, head_s, stream):
    """Single launches on row-major weights (the layout the dot-product
    variant reads) of each projection and of the lm_head with argmax at
    T = 1, 4, 8, once with the dot-product variant (v_dot2_f32_f16, lanes
    split K) and once with the matrix-core one; weight copies rotated as in
    single_launches."""
    out = {}
    hn, hk = synth.LM_HEAD
    head2 = (head_p.clone(), head_s.clone())  # two copies: 1.3 GB rotated
    try:
        for T in (1, 4, 8):
            for proj in VARIANT_SHAPES + ("lm_head",):
                if proj == "lm_head":
                    N, K = hn, hk
                    x = to_dev(synth.activations(synth.TID_LM_HEAD + 3, T, K), torch)
                    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
                    ws = torch.empty(w4a16.workspace_bytes(N, T), dtype=torch.uint8, device="cuda")
                    fns = [lambda p=p, sc=sc: w4a16.head_gather(p, sc, x, scores=True, argmax=True, out=y,
                                                                  workspace=ws, stream=stream)
                           for p, sc in ((head_p, head_s), head2)]
                else:
                    N, K = synth.PROJECTIONS[proj]
                    x = to_dev(synth.activations(synth.tid_layer(0, proj), T, K), torch)
                    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
                    fns = [lambda p=w[2], sc=w[3]: w4a16.matmul(p, sc, x, out=y, stream=stream)
                           for w in weights if w[0] == proj]
                wb = metrics.weight_bytes(N, K)
                row = {}
                for v in ("dot", "mfma"):
                    w4a16.set_variant(v)
                    us = time_rotating(torch, fns, stream)
                    row[f"{v}_us"] = round(us, 2)
                    row[f"{v}_GBps"] = round(metrics.gbps(wb, us / 1000), 1)
                out[f"{proj}_T{T}"] = row
                log(f"variant {proj} T={T}: dot {row['dot_us']:.1f} us ({row['dot_GBps']:.0f} GB/s), "
                    f"matrix core {row['mfma_us']:.1f} us ({row['mfma_GBps']:.0f} GB/s)")
    finally:
        w4a16.set_variant("auto")
    return out


def variants_pass(torch, w4a16, weights, head_p, head_s, stream):
    """Untimed: for T = 1, 4, 8, each projection (layer 0) and the lm_head
    with argmax, one launch with the dot-product variant, then one with the
    matrix-core variant (counter collection).  Returns the launch order
    (workload, calls, dispatches per call, weight bytes)."""
    hn, hk = synth.LM_HEAD
    order = []
    try:
        for T in (1, 4, 8):
            for v in ("dot", "mfma"):
                w4a16.set_variant(v)
                for proj in VARIANT_SHAPES:
                    N, K = synth.PROJECTIONS[proj]
                    w = next(w for w in weights if w[0] == proj)
                    x = to_dev(synth.activations(synth.tid_layer(0, proj), T, K), torch)
                    w4a16.matmul(w[2], w[3], x, stream=stream)
                    order.append({"workload": f"{proj} T={T} {v}", "untimed": 0, "timed": 1, "dispatches": 1,
                                  "weight_bytes": metrics.weight_bytes(N, K)})
                x = to_dev(synth.activations(synth.TID_LM_HEAD + 3, T, hk), torch)
                w4a16.head_gather(head_p, head_s, x, scores=True, argmax=True, stream=stream)
                order.append({"workload": f"lm_head T={T} {v}", "untimed": 0, "timed": 1, "dispatches": 2,
                              "weight_bytes": metrics.weight_bytes(hn, hk)})
        torch.cuda.synchronize()
    finally:
        w4a16.set_variant("auto")
    log("variants pass done: T = 1, 4, 8 x {dot, matrix core} x {qkv, o, gate_up, down, lm_head}")
    return order


def read_floors(torch, w4a16, stream):
    """For a kernel trace: the library's streaming-read kernel over buffers of
    each single-launch workload's weight bytes (8 workgroups per CU, copies
    rotated past the Infinity Cache), the floor of one launch of that size."""
    hn, hk = synth.LM_HEAD
    sizes = [("small_1024x1024", metrics.weight_bytes(*synth.SMALL))]
    sizes += [(proj, metrics.weight_bytes(*synth.PROJECTIONS[proj])) for proj in synth.PROJ_ORDER]
    sizes += [("draft_head_32768", metrics.weight_bytes(synth.DRAFT_IDS, hk)), ("lm_head", metrics.weight_bytes(hn, hk))]
    wg = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
    out = {}
    for name, nbytes in sizes:
        n = (nbytes + 15) // 16 * 16
        copies = 2 if n > (128 << 20) else 20
        bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
        fns = [lambda b=b: w4a16.stream_read(b, sink, wg, stream=stream) for b in bufs]
        us = time_rotating(torch, fns, stream, tag=f"read_floor_{name}", nbytes=n)
        out[name] = round(us, 2)
        del bufs, fns
        torch.cuda.empty_cache()
    log(f"read floors (event-timed, us): {out}")
    return out


def read_ceiling(torch, w4a16, stream, gib=4, reps=10):
    """The library's plain streaming-read kernel over a 4 GiB buffer (16-byte
    nontemporal loads, 8 workgroups per CU): the achievable read rate."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    wg = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
    for _ in range(3):
        w4a16.stream_read(src, sink, wg, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        w4a16.stream_read(src, sink, wg, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, sink
    return {"GBps": round(metrics.gbps(n, ms), 1), "bytes": n, "workgroups": wg, "ms": round(ms, 4)}


def verify_epilogue(torch, w4a16, head_y, T, stream, reps=50):
    """Per-row top-32 of the lm_head scores (two launches), greedy acceptance
    of T - 1 drafts (one launch) and the draft-head id list of 32,768 base
    ids plus 4,096 sequence ids (one launch), timed on the launch stream."""
    k = 32
    n_rows = head_y.shape[1]
    ws = torch.empty(w4a16.topk_workspace_bytes(n_rows, T, k), dtype=torch.uint8, device="cuda")
    target = torch.zeros(T, dtype=torch.int32, device="cuda")
    draft = torch.zeros(max(T - 1, 1), dtype=torch.int32, device="cuda")
    base = to_dev(synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, n_rows), torch)
    seq = to_dev(np.random.default_rng(0).integers(0, n_rows, 4096).astype(np.int32), torch)
    out = {}
    for name, fn in (("topk32_us", lambda: w4a16.topk(head_y, k, workspace=ws, stream=stream)),
                     ("greedy_us", lambda: w4a16.greedy_accept(target, draft[:T - 1] if T > 1 else None, 1, T,
                                                               stream=stream)),
                     ("draft_union_us", lambda: w4a16.draft_union(base, seq, n_rows, stream=stream))):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = round(1000.0 * e0.elapsed_time(e1) / reps, 2)
    return out


def graph_step(torch, w4a16, probs, head, reps):
    """One step as 256 matmul launches plus the lm_head call, captured once
    into a HIP graph and replayed (launch overhead off the host)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for tw, _, x, y in probs:  # warm the plans and the device check outside capture
            w4a16.matmul_tiled(tw, x, out=y)
        head(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream()
        for tw, _, x, y in probs:
            w4a16.matmul_tiled(tw, x, out=y, stream=s)
        head(s)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": round(e0.elapsed_time(e1) / reps, 4), "launches": len(probs) + 2}


def plain_launch_step(torch, w4a16, probs, head, stream, reps):
    """One step as 256 matmul calls plus the lm_head call, each a separate
    launch issued from the host on one stream (no graph)."""
    def one():
        for tw, _, x, y in probs:
            w4a16.matmul_tiled(tw, x, out=y, stream=stream)
        head(stream)
    for _ in range(3):
        one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        one()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"ms_per_step": round(e0.elapsed_time(e1) / reps, 4), "launches": len(probs) + 2}


def cpu_baseline(T, target_s, step_out=None):
    """The oracle (plain C, fp64) on the host cores, on whole layers of the same
    pass until about target_s seconds of work, reported as weight GB/s; then,
    with step_out (host copies of the last timed step's outputs), the parity
    of that step against the oracle (step_parity)."""
    import oracle

    threads = oracle.default_threads()
    done_bytes = 0
    spent = 0.0
    layers = 0
    for layer in range(synth.LAYERS):
        for proj in synth.PROJ_ORDER:
            N, K = synth.PROJECTIONS[proj]
            p, s = synth.weight(synth.tid_layer(layer, proj), N, K)
            x = synth.activations(synth.tid_layer(layer, proj), T, K)
            t = time.time()
            oracle.matmul(p, s, x, nthreads=threads, want_abs=False)
            spent += time.time() - t
            done_bytes += metrics.weight_bytes(N, K)
        layers += 1
        if spent >= target_s:
            break
    g = done_bytes / spent / 1e9
    log(f"CPU oracle: {layers} layers at T={T} in {spent:.1f} s on {threads} threads: {g:.3f} GB/s")
    # the same oracle on one thread, on the qkv projection of layer 0
    N, K = synth.PROJECTIONS["qkv"]
    p, s = synth.weight(synth.tid_layer(0, "qkv"), N, K)
    x = synth.activations(synth.tid_layer(0, "qkv"), T, K)
    t = time.time()
    oracle.matmul(p, s, x, nthreads=1, want_abs=False)
    t1 = time.time() - t
    g1 = metrics.weight_bytes(N, K) / t1 / 1e9
    log(f"CPU oracle, one thread: layer 0 qkv at T={T} in {t1:.1f} s: {g1:.4f} GB/s")
    out = {"value": round(g, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{layers} of 64 layers (qkv, o, gate_up, down) at T={T}, fp64 oracle, {spent:.1f} s",
           "single_thread": {"value": round(g1, 4), "unit": "GB/s", "cores": 1,
                             "sample": f"layer 0 qkv at T={T}, {t1:.1f} s"}}
    if step_out is not None:
        out["parity"] = step_parity(oracle, T, step_out)
    return out


def step_parity(oracle, T, step_out):
    """The timed step's outputs against the oracle (after the timing): every
    output of layer 0's four projections and every lm_head score, as the
    largest |y_gpu - y_ref| / (1e-3 * sum_k |w*x| + 1e-6) (at most 1 passes),
    and each row's argmax id against the oracle's, exact unless the oracle's
    gap between its best and its best other id is below the GPU's error on
    those two rows (a near tie, counted)."""
    worst = 0.0

    def ratio(y_gpu, y_ref, a_ref):
        return float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref) / (1e-3 * a_ref + 1e-6)))

    for proj, y_gpu in step_out["layer0"]:
        N, K = synth.PROJECTIONS[proj]
        p, s = synth.weight(synth.tid_layer(0, proj), N, K)
        x = synth.activations(synth.tid_layer(0, proj), T, K)
        worst = max(worst, ratio(y_gpu, *oracle.matmul(p, s, x)))
    hn, hk = synth.LM_HEAD
    hp, hs = synth.weight(synth.TID_LM_HEAD, hn, hk)
    hx = synth.activations(synth.TID_LM_HEAD, T, hk)
    y_ref, a_ref = oracle.matmul(hp, hs, hx)
    y_gpu = step_out["head_y"]
    worst = max(worst, ratio(y_gpu, y_ref, a_ref))
    ref_id, _, gap = oracle.argmax(y_ref)
    ids = step_out["head_id"]
    exact = int(np.sum(ids == ref_id))
    near = 0
    for t in range(T):
        if ids[t] != ref_id[t] and ids[t] >= 0:
            i, j = int(ids[t]), int(ref_id[t])
            err = abs(float(y_gpu[t, i]) - y_ref[t, i]) + abs(float(y_gpu[t, j]) - y_ref[t, j])
            near += int(gap[t] < err)
    log(f"parity of the timed step: max err / tol {worst:.3g}; argmax {exact}/{T} exact, {near} near tie(s)")
    return {"max_err_over_tol": float(f"{worst:.3g}"), "argmax_match": f"{exact}/{T}", "argmax_near_ties": near,
            "checked": "every output of layer 0's qkv, o, gate_up and down and every lm_head score of the last "
                       "timed step; the argmax id of each of its rows"}


if __name__ == "__main__":
    main()
