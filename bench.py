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
LLC_BYTES = 256 * 1024 * 1024  # MI355X last-level (Infinity) cache
# MI355X dense MFMA peaks, AMD's published figures (TFLOP/s)
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
METRIC = "scan elements/s and achieved HBM GB/s vs MI355X peak (rocprof), per config"
# Every file whose code shapes what the kernels do: the kernels, their shared headers and the
# host code that picks kernels and launch shapes.
KERNEL_SOURCES = ["scan_primitives_amd/csrc/element_scan.hip", "scan_primitives_amd/csrc/normcap_quad.hip",
                  "scan_primitives_amd/csrc/matrix_scan.hip", "scan_primitives_amd/csrc/matrix_scan_grad.hip",
                  "scan_primitives_amd/csrc/table_scan.hip", "scan_primitives_amd/csrc/ms_mfma.hpp",
                  "scan_primitives_amd/csrc/sx_common.hpp", "scan_primitives_amd/csrc/sx_api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def git_sha() -> str | None:
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


def code_only(text: str) -> str:
    """C/C++ source with its comments removed and blank lines dropped, so that
    a change to comments alone keeps the hash below (string and character
    literals are kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            k = text.find("*/", i + 2)
            i = n if k < 0 else k + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash() -> str:
    """First 16 hex digits of the sha256 of KERNEL_SOURCES' code (comments removed)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
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


def mfma_figures(w, sec: float) -> dict:
    """Matrix-scan MFMA utilisation for one call taking ``sec`` seconds.

    Algorithmic: the recurrence's own work, one n x n by n x m product a step
    (2 n^2 m flops), against the f32 MFMA peak (the scan computes in f32 for f32
    and bf16 operands alike). Executed: the MFMA operations the kernels issue
    per call, from the committed rocprofv3 counter summary (SQ_INSTS_VALU_MFMA_
    MOPS_*) when it was taken on the current kernel sources, against each
    precision's own peak; null otherwise."""
    if w.op != "matrix_scan":
        return {}
    b = w.tensors["b"]
    n, m = int(b.shape[-2]), int(b.shape[-1])
    steps = b.numel() // (n * m)
    alg = 2.0 * n * n * m * steps / sec / 1e12
    out = {"mfma_algorithmic_tflops": round(alg, 3),
           "mfma_algorithmic_util": round(alg / MFMA_PEAK_TFLOPS["f32"], 5),
           "mfma_executed": None}
    path = os.path.join(ROOT, "profiles", "mfma.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return out
    if data.get("kernel_source_hash") != kernel_source_hash():
        return out
    counted = data.get("per_call", {}).get(w.name)
    if counted:
        ex = {}
        for prec, flops in counted.items():
            tf = flops / sec / 1e12
            ex[prec] = {"tflops": round(tf, 3), "util": round(tf / MFMA_PEAK_TFLOPS[prec], 5)}
        out["mfma_executed"] = ex
    return out


def _oracle_call(w_op, w_body, w_axis, w_state_axis, w_reverse, arrays):
    import oracle
    if w_op == "element_scan":
        return oracle.element_scan(w_body, arrays["initial"], [arrays["x"], arrays["s"]], axis=w_axis,
                                   state_axis=w_state_axis, reverse=w_reverse)
    return oracle.matrix_scan(arrays["a"], arrays["b"], axis=w_axis, reverse=w_reverse)


# CPU baseline workers (spawned processes): the inputs sit in shared memory, one
# block per array, and a task names a workload and a slice of its batch dim (dim
# 0; the scans run along dim 1, so a slice is an independent sub-problem).
_SHARED = {}


def _oracle_worker_init(specs):
    from multiprocessing import shared_memory

    import numpy as np
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)  # one core per worker
    for key, (name, shape, dtype) in specs.items():
        shm = shared_memory.SharedMemory(name=name)
        _SHARED[key] = (shm, np.ndarray(shape, dtype=dtype, buffer=shm.buf))


def _oracle_worker_task(task):
    j, meta, names, lo, hi = task
    arrays = {k: _SHARED[(j, k)][1][lo:hi] for k in names}
    _oracle_call(*meta, arrays)
    return 0


def cpu_baseline(workloads, min_seconds: float = 10.0) -> dict:
    """Time the CPU oracle, as it stands, on the same workloads, on 1 core and
    on the machine's cores (at most 16, the CPU share of one GPU on the box): whole
    passes over every workload at full size, repeated until at least
    ``min_seconds`` have been spent each way. The multi-core passes split each
    workload's batch dim across worker processes (the oracle itself is
    unchanged); the inputs are shared, not copied per pass."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import numpy as np
    from threadpoolctl import threadpool_limits

    hosts = [{k: np.ascontiguousarray(v.float().numpy()) for k, v in w.tensors.items()} for w in workloads]
    metas = [(w.op, getattr(w, "body", None), w.axis, w.state_axis, w.reverse) for w in workloads]
    elems_per_pass = sum(w.out_numel for w in workloads)

    # 1 core, after one untimed pass (first-touch and import costs stay out, as for the workers)
    one_s, one_passes = 0.0, 0
    with threadpool_limits(limits=1):
        for meta, host in zip(metas, hosts):
            _oracle_call(*meta, host)
        while one_passes == 0 or one_s < min_seconds:
            for meta, host in zip(metas, hosts):
                t0 = time.perf_counter()
                _oracle_call(*meta, host)
                one_s += time.perf_counter() - t0
            one_passes += 1
    one_rate = one_passes * elems_per_pass / one_s

    # the machine's cores: worker processes over shared inputs
    cores = max(1, min(16, os.cpu_count() or 1))
    blocks, specs = [], {}
    try:
        for j, host in enumerate(hosts):
            for k, arr in host.items():
                shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
                np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
                blocks.append(shm)
                specs[(j, k)] = (shm.name, arr.shape, arr.dtype.str)
        tasks = []
        for j, (w, host) in enumerate(zip(workloads, hosts)):
            lead = next(iter(host.values())).shape[0]
            cuts = np.linspace(0, lead, min(cores, lead) + 1).astype(int)
            names = list(host.keys())
            tasks += [(j, metas[j], names, int(lo), int(hi)) for lo, hi in zip(cuts[:-1], cuts[1:]) if hi > lo]
        with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn"),
                                 initializer=_oracle_worker_init, initargs=(specs,)) as pool:
            list(pool.map(_oracle_worker_task, tasks))  # start the workers, warm them up
            many_s, many_passes = 0.0, 0
            while many_passes == 0 or many_s < min_seconds:
                t0 = time.perf_counter()
                list(pool.map(_oracle_worker_task, tasks))
                many_s += time.perf_counter() - t0
                many_passes += 1
    finally:
        for shm in blocks:
            shm.close()
            shm.unlink()
    many_rate = many_passes * elems_per_pass / many_s
    log(f"cpu oracle: {one_rate:.3e} elements/s on 1 core, {many_rate:.3e} on {cores} cores")
    return {"value": many_rate, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "single_core_value": one_rate,
            "sample": f"the float64 numpy oracle over every selected workload at full size: {one_passes} passes on "
                      f"1 core ({one_s:.1f} s) and {many_passes} passes on {cores} worker processes, each workload's "
                      f"batch dim split across them ({many_s:.1f} s wall); os.cpu_count() = {os.cpu_count()}"}


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
        entry = {
            "workload": w.name,
            "call_us": round(sec * 1e6, 3),
            "calls_per_replay": r,
            "elements_per_s": w.out_numel / sec,
            "algorithmic_bytes": w.algorithmic_bytes,
            "hbm_gbs": round(gbs, 2),
            "hbm_frac_warm": round(gbs / HBM_PEAK_GBS, 4),
            "in_step": j < len(workloads),
        }
        entry.update(mfma_figures(w, sec))
        per_config.append(entry)
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
        # the quoted HBM fraction: cold for a workload that fits the last-level cache (its warm
        # figure would measure that cache), warm (back-to-back calls) otherwise
        fits = w.algorithmic_bytes <= LLC_BYTES
        per_config[j]["hbm_frac"] = per_config[j]["hbm_frac_cold" if fits else "hbm_frac_warm"]
        per_config[j]["hbm_frac_basis"] = "cold" if fits else "warm"
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
    roofline = {"bound": "hbm", "achieved": round(dc["hbm_frac"] * HBM_PEAK_GBS, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": dc["hbm_frac"], "traffic": measured_traffic(dw.name), "kernel": dw.name,
                "basis": dc["hbm_frac_basis"], "algorithmic_bytes_per_call": dw.algorithmic_bytes}

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
