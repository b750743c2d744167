"""Throughput of the scan library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only 0,2,...]
                    [--no-cpu-baseline] [--with-copy] [--eager] [--no-extra]

One step runs the whole hot path once: the five standard workloads of
``scan_primitives_amd.workloads`` (tanh-affine, norm-cap, reverse max-plus,
matrix-scan f32 m=1, matrix-scan bf16 m=16 reverse), each as one library
call on inputs already resident in HBM. The step is captured once in a HIP
graph (the library launches on torch's current stream, which is the capture
stream), so host-side launch work stays out of the timed region; W untimed
replays come first, then K timed replays bracketed by device synchronisation.

Each workload's call is also timed on its own: a graph of R back-to-back
calls (R >= 16, and enough calls that a replay moves at least 32 MiB, up to
64), replayed K times between two HIP events on the capture stream; the
per-call time is the elapsed time over K * R, so the few microseconds a graph
launch costs are spread over R calls. A cold figure follows: the median of
single calls, each after a 512 MiB write that evicts the last-level cache
(256 MB), timed between HIP events (it includes the launch). This gives each workload's elements/s, algorithmic GB/s and
fraction of the 8 TB/s HBM peak.

linear-scan and cumsum ([64,4096,256] f32 along axis 1), the gradients of
the five workloads, the f32 matrix workload with :projective and table-scan
on [4096,16384] int32 symbols are timed the same two ways and reported in
``per_config`` with ``"in_step": false``; they are not part of the step or
of ``value`` (``--no-extra`` skips them).

Prints ONE JSON line on stdout. ``value`` is output elements per second over
the timed steps; ``per_config`` has each workload's figures; ``roofline``
describes the call that takes the most time; ``cpu_baseline`` is the CPU
oracle timed on the same workloads on the host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
METRIC = "scan elements/s and achieved HBM GB/s vs MI355X peak (rocprof), per config"
KERNEL_SOURCES = ["scan_primitives_amd/csrc/element_scan.hip", "scan_primitives_amd/csrc/normcap_quad.hip",
                  "scan_primitives_amd/csrc/matrix_scan.hip", "scan_primitives_amd/csrc/matrix_scan_grad.hip",
                  "scan_primitives_amd/csrc/table_scan.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def git_sha() -> str | None:
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_label: str):
    """HBM bytes per call from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("per_call", {}).get(kernel_label)
    return None if entry is None else entry.get("bytes")


def cpu_baseline(workloads, min_seconds: float = 10.0) -> dict:
    """Time the CPU oracle, as it stands, on the same workloads: whole passes
    over every workload at full size, repeated until at least ``min_seconds``
    of oracle time have been spent (one pass takes well under a second)."""
    from threadpoolctl import threadpool_limits

    import oracle

    total_elems, total_s, passes = 0, 0.0, 0
    hosts = [{k: v.float().numpy() for k, v in w.tensors.items()} for w in workloads]
    with threadpool_limits(limits=1):
        while passes == 0 or total_s < min_seconds:
            for w, host in zip(workloads, hosts):
                t0 = time.perf_counter()
                if w.op == "element_scan":
                    oracle.element_scan(w.body, host["initial"], [host["x"], host["s"]], axis=w.axis,
                                        state_axis=w.state_axis, reverse=w.reverse)
                else:
                    oracle.matrix_scan(host["a"], host["b"], axis=w.axis, reverse=w.reverse)
                dt = time.perf_counter() - t0
                if passes == 0:
                    log(f"cpu oracle {w.name}: {dt:.3f} s")
                total_elems += w.out_numel
                total_s += dt
            passes += 1
    return {"value": total_elems / total_s, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} passes of the float64 numpy oracle over every selected workload at full size, "
                      f"single-threaded; {total_elems} output elements in {total_s:.2f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", type=str, default=None, help="comma-separated workload indices 0..4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-copy", action="store_true",
                    help="also run a plain 256 MiB device copy per step (reference kernel for PMC byte counts)")
    ap.add_argument("--eager", action="store_true", help="launch calls directly instead of replaying graphs")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the linear-scan, cumsum and gradient calls timed beside the step")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scans shard with no or one small exchange, see the design notes)", file=sys.stderr)
        return 2

    import torch

    import scan_primitives_amd as sx
    from scan_primitives_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 3
    sx.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    which = None if args.only is None else [int(i) for i in args.only.split(",")]
    workloads = W.standard_workloads(which)
    extras = [] if args.no_extra else W.extra_workloads()
    log("generated inputs: " + "; ".join(w.name for w in workloads + extras))
    resident = [w.on(dev) for w in workloads]
    resident_extra = [w.on(dev) for w in extras]
    for w, t in zip(extras, resident_extra):  # the forward result a gradient reads, computed once here
        if w.op == "matrix_scan_backward":
            t["h"] = sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse)
        elif w.op == "element_scan_backward":
            t["h"] = sx.element_scan(w.body, t["initial"], [t["x"], t["s"]], axis=w.axis, state_axis=w.state_axis,
                                     reverse=w.reverse)
    torch.cuda.synchronize()

    def call(w, t):
        if w.op == "element_scan":
            return sx.element_scan(w.body, t["initial"], [t["x"], t["s"]], axis=w.axis, state_axis=w.state_axis,
                                   reverse=w.reverse)
        if w.op == "linear_scan":
            return sx.linear_scan(t["a"] if "a" in t else w.meta["a_number"], t["b"], axis=w.axis,
                                  reverse=w.reverse, out_dtype=w.out_dtype)
        if w.op == "matrix_scan_backward":
            return sx.matrix_scan_backward(t["a"], tuple(t["b"].shape), t["h"], t["g"], axis=w.axis,
                                           reverse=w.reverse)
        if w.op == "table_scan":
            return sx.table_scan(t["table"], t["symbols"], axis=w.axis, start=w.meta.get("start", 0))
        if w.op == "element_scan_backward":
            return sx.element_scan_backward(w.body, t["initial"], [t["x"], t["s"]], t["h"], t["g"], axis=w.axis,
                                            state_axis=w.state_axis, reverse=w.reverse)
        return sx.matrix_scan(t["a"], t["b"], axis=w.axis, reverse=w.reverse, out_dtype=w.out_dtype,
                              projective=w.meta.get("projective", False))

    copy_src = copy_dst = None
    if args.with_copy:
        copy_src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        copy_dst = torch.empty_like(copy_src)

    def one_step():
        for w, t in zip(workloads, resident):
            call(w, t)
        if copy_src is not None:
            copy_dst.copy_(copy_src)

    # eager warm-up (also sizes the caching allocator), then capture
    for _ in range(2):
        one_step()
        for w, t in zip(extras, resident_extra):
            call(w, t)
    torch.cuda.synchronize()
    # every measured call: the step's workloads, then the extra ones (not part of the step)
    timed = workloads + extras
    timed_inputs = resident + resident_extra
    reps = [max(16, min(64, math.ceil((32 << 20) / w.algorithmic_bytes))) for w in timed]
    graphs, step_graph, keep = [], None, []
    if not args.eager:
        for w, t, r in zip(timed, timed_inputs, reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                keep.append([call(w, t) for _ in range(r)])
            graphs.append(g)
        step_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(step_graph):
            one_step()
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    # ---- per-workload call time: K replays of a graph of R calls, between two events
    per_config = []
    for j, (w, t, r) in enumerate(zip(timed, timed_inputs, reps)):
        def run_once():
            if args.eager:
                for _ in range(r):
                    call(w, t)
            else:
                graphs[j].replay()
        for _ in range(args.warmup):
            run_once()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            run_once()
        e1.record(stream)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / (args.steps * r)
        gbs = w.algorithmic_bytes / sec / 1e9
        per_config.append({
            "workload": w.name,
            "call_us": round(sec * 1e6, 3),
            "calls_per_replay": r,
            "elements_per_s": w.out_numel / sec,
            "algorithmic_bytes": w.algorithmic_bytes,
            "hbm_gbs": round(gbs, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "in_step": j < len(workloads),
        })
        log(f"{w.name}: {sec * 1e6:.2f} us/call, {w.out_numel / sec:.3e} elements/s, {gbs:.1f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")

    # ---- the same calls cold: before each one, a 512 MiB write evicts the 256 MB last-level cache
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=dev)
    for j, (w, t) in enumerate(zip(timed, timed_inputs)):
        times = []
        for _ in range(max(args.steps, 20)):
            flush.fill_(float(j))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(w, t)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        times.sort()
        sec = times[len(times) // 2]
        gbs = w.algorithmic_bytes / sec / 1e9
        per_config[j]["call_us_cold"] = round(sec * 1e6, 3)
        per_config[j]["hbm_frac_cold"] = round(gbs / HBM_PEAK_GBS, 4)
        log(f"{w.name} (cold, median of {len(times)} single calls): {sec * 1e6:.2f} us/call, {gbs:.1f} GB/s")
    del flush

    # ---- whole job: K steps, each one pass over every workload
    for _ in range(args.warmup):
        one_step() if args.eager else step_graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step() if args.eager else step_graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_elems = sum(w.out_numel for w in workloads) * args.steps
    log(f"{args.steps} steps in {wall * 1e3:.2f} ms")

    dom = max(range(len(workloads)), key=lambda j: per_config[j]["call_us"])
    dw, dc = workloads[dom], per_config[dom]
    roofline = {"bound": "hbm", "achieved": dc["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dc["hbm_frac"], "traffic": measured_traffic(dw.name), "kernel": dw.name,
                "algorithmic_bytes_per_call": dw.algorithmic_bytes}

    result = {
        "metric": METRIC,
        "value": total_elems / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": " + ".join(w.name for w in workloads), "commit": git_sha(),
                   "kernel_source_hash": kernel_source_hash(), "timing": "eager" if args.eager else "hip-graph"},
        "roofline": roofline,
        "per_config": per_config,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(workloads)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
