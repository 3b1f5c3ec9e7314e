"""Benchmark of the MI355X Fast LapSum soft top-k (forward + backward).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs extreme,attack,...]

One step = one forward (threshold b and probabilities p) plus one backward
(dr, dk) over one batch, inputs resident in HBM.  The 1e8 rows time K steps;
the other workloads at least 1000 (their steps take microseconds, and the
first launch and the closing synchronisation are paid once).  The headline workload is
the single row of 1e8 scores (mixture 0.9 N(0,1) + 0.1 N(3, 0.5), k = 1e5,
t = 0.01, bracketing path); the other workloads are reported beside it, each
with its step-time distribution, the oracle timed on the host cores, the
bracketing hit rate where it applies and the budget drift of DFTopK's fixed
midpoint threshold.  Prints ONE JSON line.

Byte model (algorithmic bytes per score, what the method itself must move):
  on-chip rows:        fwd 8 (r in, p out), bwd 12 (g, p in, dr out)
  bracketing:          fwd 12 (r read by the filter pass and the apply pass, p out),
                       bwd 20 (g, p read twice, dr out: dk needs the whole row)
  bucket, sort and bisection rows: fwd 8 compulsory (sort and bisection
                       traffic measured, not credited), bwd 20
Per-kernel algorithmic bytes: filter 4, apply 8, bwd_reduce 8, bwd_apply 12,
on-chip fwd 8, on-chip bwd 12 (x scores per launch).
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # MI355X HBM3E, bytes/s
MALL_BYTES = 256 << 20

STAGE_BYTES = {"onchip_fwd": 8, "filter": 4, "apply": 8, "onchip_bwd": 12, "bwd_reduce": 8, "bwd_apply": 12}
KERNEL_NAMES = {"onchip_fwd": "onchip_forward_wave", "filter": "filter_kernel", "apply": "apply_kernel",
                "onchip_bwd": "onchip_backward_wave", "bwd_reduce": "bwd_reduce_kernel",
                "bwd_apply": "bwd_apply_kernel", "band": "band_solve_onchip / band_*_kernel",
                "select": "select_bucket_kernel", "sample": "sample_kernel", "bucket": "band_*_kernel",
                "init": "init_rows_kernel", "sort": "rsort_*_kernel", "solve": "rsort_agg/locate_kernel",
                "bisect": "bisect_*_kernel"}


class Hip:
    """HIP events through the runtime (torch already loaded libamdhip64).

    Events are recycled, never destroyed: after a few thousand events had
    been created and destroyed in one process (the per-stage instrumentation
    of several workloads), recording an event was measured to cost about a
    whole GPU round trip (a backward pass of 15 us took 0.35 ms per step
    with two event records), which would distort every later timed loop.
    destroy() returns events to the pool; they are only reused after the
    caller has synchronised on them."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.free = []

    def event(self):
        if self.free:
            return self.free.pop()
        ev = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs):
        self.free.extend(e for e in evs if e)


WORKLOADS = {
    # name: generator, path, algorithmic bytes per score fwd / bwd
    "extreme": dict(gen="extreme", path="auto", fwd_b=12, bwd_b=20),
    "attack": dict(gen="attack", path="auto", fwd_b=12, bwd_b=20),
    "routing": dict(gen="routing", path="auto", fwd_b=8, bwd_b=12),
    # the routing batch with a budget and a temperature per row (k_i in [2, 14],
    # t_i log-uniform in [0.02, 0.1], seed 4700)
    "routing_per_row": dict(gen="routing", path="auto", fwd_b=8, bwd_b=12, per_row=True),
    "coder_bracket": dict(gen="coder", path="bracket", fwd_b=12, bwd_b=20),
    "coder_bucket": dict(gen="coder", path="bucket", fwd_b=8, bwd_b=20),
    "coder_sort": dict(gen="coder", path="sort", fwd_b=8, bwd_b=20),
    "coder_bisect": dict(gen="coder", path="bisect", fwd_b=8, bwd_b=20),
    # the 1e8 row through the other exact solvers: the pages compare
    # bracketing with a full sort at this size, and the full sort with
    # per-query bisection
    "extreme_bucket": dict(gen="extreme", path="bucket", fwd_b=8, bwd_b=20),
    "extreme_sort": dict(gen="extreme", path="sort", fwd_b=8, bwd_b=20),
    "extreme_bisect": dict(gen="extreme", path="bisect", fwd_b=8, bwd_b=20),
    "tiny": dict(gen="tiny", path="auto", fwd_b=8, bwd_b=12),
}
DEFAULT_CONFIGS = ("extreme,attack,routing,routing_per_row,coder_bracket,coder_bucket,coder_sort,coder_bisect,"
                   "extreme_bucket,extreme_sort,extreme_bisect,tiny")

# Bracketing hit-rate trials (seeds) per workload: 100 x 32 rows for the
# coder batch, 1000 for the attack row, 100 for the 1e8 row.
HIT_TRIALS = {"coder": 100, "attack": 1000, "extreme": 100}

# CPU oracle baseline per workload: threads and runs (median), and for the
# 1e8 row a bounded prefix sample (the oracle's bisection runs at ~2e5
# scores/s on one core, so the full row would take about ten minutes).
# Batches use every host core, single rows one core; about 30 s in all.
CPU_PLAN = {"tiny": dict(threads="all", runs=3), "routing": dict(threads="all", runs=3),
            "coder": dict(threads="all", runs=3), "attack": dict(threads=1, runs=1),
            "extreme": dict(threads=1, runs=1, prefix=5_000_000)}

_WORKLOAD_CACHE = {}


def workload(gen):
    """Each generator's arrays once per run (the 1e8 row takes seconds to draw)."""
    from sparse_selection_primitive_amd import workloads
    if gen not in _WORKLOAD_CACHE:
        _WORKLOAD_CACHE[gen] = workloads.by_name(gen)
    return _WORKLOAD_CACHE[gen]


def quantiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90))}


# Source files each streaming kernel is compiled from (a change to any of them
# invalidates the HBM traffic counters recorded for that kernel).
_COMMON_SRC = ["lapsum_device.hpp", "lapsum_internal.hpp"]
KERNEL_SOURCES = {"filter": ["bracket.hip", "filter_dev.hpp"] + _COMMON_SRC,
                  "apply": ["stream.hip"] + _COMMON_SRC,
                  "bwd_reduce": ["stream.hip"] + _COMMON_SRC,
                  "bwd_apply": ["stream.hip"] + _COMMON_SRC,
                  "onchip_fwd": ["onchip.hip", "segment_dev.hpp"] + _COMMON_SRC,
                  "onchip_bwd": ["onchip.hip", "segment_dev.hpp"] + _COMMON_SRC}


def source_sha(files=None) -> str:
    """Hash of the kernel sources (all of csrc/ unless `files` names some)."""
    csrc = os.path.join(ROOT, "sparse_selection_primitive_amd", "csrc")
    paths = sorted(glob.glob(os.path.join(csrc, "*"))) if files is None else [os.path.join(csrc, f) for f in files]
    h = hashlib.sha256()
    for f in paths:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stages_of(L, plan, n):
    """Stage ids a call with this plan records (forward, then backward)."""
    path = plan["path"]
    bis_stream = n > 16384
    fwd = {L.PATH_ONCHIP: [L.STAGE_ONCHIP_FWD],
           L.PATH_BUCKET: [L.STAGE_INIT, L.STAGE_BUCKET, L.STAGE_APPLY],
           L.PATH_BRACKET: [L.STAGE_SAMPLE, L.STAGE_SELECT, L.STAGE_FILTER, L.STAGE_BAND,
                            L.STAGE_APPLY],  # the fallback runs inside the band stage
           L.PATH_SORT: [L.STAGE_INIT, L.STAGE_SORT, L.STAGE_SOLVE, L.STAGE_APPLY],
           L.PATH_BISECT: [L.STAGE_INIT, L.STAGE_BISECT] + ([L.STAGE_APPLY] if bis_stream else [])}[path]
    bwd = [L.STAGE_ONCHIP_BWD] if n <= 1024 else [L.STAGE_BWD_REDUCE, L.STAGE_BWD_APPLY]
    return fwd + bwd


def bench_workload(L, hip, torch, name, spec, steps, warmup, seed=0, live_dominant=True):
    """live_dominant: time the dominant kernel with an event pair inside the
    timed region (the headline workload, run first); otherwise its time comes
    from the instrumented pass and the timed region records no per-kernel
    event (event records were measured to turn into GPU round trips late in a
    long run of workloads, inflating their timed loops several times over).
    The step-time distribution comes from one event per chunk of steps (one
    step per chunk when a step is long, enough steps for ~0.2 ms otherwise)."""
    import numpy as np
    w = workload(spec["gen"])
    rows, n = w.rows, w.n
    elems = rows * n
    set_bytes = 4 * 4 * elems
    nsets = max(1, min(16, -(-2 * MALL_BYTES // set_bytes)))  # rotate past the 256 MB Infinity Cache
    dev = torch.device("cuda:0")
    r0 = torch.from_numpy(w.r).to(dev)
    g0 = torch.from_numpy(w.g).to(dev)
    sets = []
    for i in range(nsets):
        r = r0 if i == 0 else r0.clone()
        g = g0 if i == 0 else g0.clone()
        p = torch.empty_like(r)
        b = torch.empty(rows, dtype=torch.float64, device=dev)
        dr = torch.empty_like(r)
        dk = torch.empty(rows, dtype=torch.float32, device=dev)
        sets.append((r, g, p, b, dr, dk))
    path = spec["path"]
    plan = L.plan(rows, n, w.k, w.t, path=path, seed=seed)
    k_rows = t_rows = None
    if spec.get("per_row"):
        gk = np.random.Generator(np.random.PCG64(4700))
        k_rows = torch.from_numpy(gk.uniform(2.0, 14.0, rows)).to(dev)
        t_rows = torch.from_numpy(np.exp(gk.uniform(np.log(0.02), np.log(0.1), rows))).to(dev)
    op = L.Operator(rows, n, w.k, w.t, device=dev, path=path, seed=seed, k_rows=k_rows, t_rows=t_rows)

    def step(i, ev=None):
        r, g, p, b, dr, dk = sets[i % nsets]
        op.forward(r, p, b, ev)
        op.backward(g, p, b, dr, dk, ev)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # instrumented pass: per-stage durations (not part of the timed region)
    n_inst = min(steps, 20)
    stage_ms = {}
    evsets = []
    for i in range(n_inst):
        evs = [hip.event() for _ in range(2 * L.STAGE_COUNT)]
        evsets.append(evs)
        step(i, evs)
    torch.cuda.synchronize()
    ran = stages_of(L, plan, n)
    for evs in evsets:
        for s_ in ran:
            ms = hip.elapsed_ms(evs[2 * s_], evs[2 * s_ + 1])
            stage_ms.setdefault(L.STAGE_NAMES[s_], []).append(ms)
        hip.destroy(evs)
    stage_avg = {k: sum(v) / len(v) for k, v in stage_ms.items()}
    dominant = max((k for k in stage_avg if k in STAGE_BYTES), key=lambda k: stage_avg[k])
    dom_id = L.STAGE_NAMES.index(dominant)
    est_step_ms = max(sum(stage_avg.values()), 1e-3)
    chunk = max(1, int(round(0.2 / est_step_ms)))
    chunk = min(chunk, max(1, steps // 10))

    # timed region: K steps; events only around the dominant kernel (headline)
    # and at chunk boundaries (on the stream every call is launched on)
    dom_events = [(hip.event(), hip.event()) for _ in range(steps)] if live_dominant else []
    ev_lists = []
    for a, b_ in dom_events:
        evs = [None] * (2 * L.STAGE_COUNT)
        evs[2 * dom_id], evs[2 * dom_id + 1] = a, b_
        ev_lists.append(evs)
    stream = torch.cuda.current_stream(dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps // chunk + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(steps):
        step(i, ev_lists[i] if live_dominant else None)
        if (i + 1) % chunk == 0:
            marks[(i + 1) // chunk].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [marks[j].elapsed_time(marks[j + 1]) / chunk for j in range(len(marks) - 1)]
    if live_dominant:
        dom_ms = [hip.elapsed_ms(a, b_) for a, b_ in dom_events]
        hip.destroy([e for pair in dom_events for e in pair])
        dom_avg = sum(dom_ms) / len(dom_ms)
    else:
        dom_avg = stage_avg[dominant]

    # the same steps replayed from one HIP graph that holds a forward+backward
    # on every buffer set in turn: the launch cost of each kernel leaves the
    # step, and one graph launch covers nsets steps (a graph launch per
    # ~20 us step would leave the GPU waiting on the host)
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gr, stream=cap):
            cs = cap.cuda_stream
            for i in range(nsets):
                r, g, p, b, dr, dk = sets[i]
                op.forward(r, p, b, stream=cs)
                op.backward(g, p, b, dr, dk, stream=cs)
    torch.cuda.current_stream(dev).wait_stream(cap)
    for _ in range(max(1, warmup // nsets)):
        gr.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // nsets))
    t2 = time.perf_counter()
    for _ in range(reps):
        gr.replay()
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t2
    graph_steps = reps * nsets
    del gr

    # forward-only timing (same rotation)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        r, g, p, b, dr, dk = sets[i % nsets]
        op.forward(r, p, b)
    torch.cuda.synchronize()
    wall_fwd = time.perf_counter() - t1

    ms_step = 1e3 * wall / steps
    ms_fwd = 1e3 * wall_fwd / steps
    ms_graph = 1e3 * wall_graph / graph_steps
    step_bytes = (spec["fwd_b"] + spec["bwd_b"]) * elems
    dom_bytes = STAGE_BYTES[dominant] * elems
    path_name = ["auto", "onchip", "bucket", "bracket", "sort", "bisect"][plan["path"]]
    out = {
        "workload": w.name, "rows": rows, "n": n, "k": w.k, "t": w.t, "path": path_name,
        "fwd_bwd_elements_per_s": elems / (ms_step * 1e-3),
        "fwd_elements_per_s": elems / (ms_fwd * 1e-3),
        "ms_per_step": ms_step, "ms_fwd": ms_fwd,
        "step_ms_quantiles": {**quantiles(per_step), "chunk_steps": chunk, "chunks": len(per_step)},
        "hbm_fraction_step": step_bytes / (ms_step * 1e-3) / HBM_PEAK,
        "hbm_fraction_fwd": spec["fwd_b"] * elems / (ms_fwd * 1e-3) / HBM_PEAK,
        "ms_per_step_graph": ms_graph,
        "fwd_bwd_elements_per_s_graph": elems / (ms_graph * 1e-3),
        "hbm_fraction_step_graph": step_bytes / (ms_graph * 1e-3) / HBM_PEAK,
        "bytes_per_element_fwd_bwd": spec["fwd_b"] + spec["bwd_b"],
        "buffer_sets": nsets,
        "stage_ms": {k: round(v, 5) for k, v in stage_avg.items()},
        "dominant": {"stage": dominant, "kernel": KERNEL_NAMES[dominant], "avg_ms": dom_avg,
                     "bytes": dom_bytes, "GBps": dom_bytes / (dom_avg * 1e-3) / 1e9,
                     "timing": "events in the timed region" if live_dominant else "instrumented pass"},
    }
    if plan["path"] == L.PATH_BRACKET:
        out["bracket"] = {"m": plan["m"], "lo": plan["lo"], "hi": plan["hi"], "band_capacity": plan["band_capacity"]}
    if spec.get("per_row"):
        out["workload"] = w.name + "_per_row_k_t"
        out["k"], out["t"] = "per row, uniform in [2, 14]", "per row, log-uniform in [0.02, 0.1]"
    return out


def hit_rate(L, torch, gen, trials):
    """Rows certified at the first bracket over `trials` sample seeds."""
    w = workload(gen)
    r = torch.from_numpy(w.r).cuda()
    hits = total = widened = 0
    bands = []
    for seed in range(trials):
        _, _, st = L.lapsum_forward(r, w.k, w.t, path="bracket", seed=1000 + seed, stats=True)
        fl = st["flags"]
        hits += int(((fl & L.FLAG_HIT) != 0).sum().item())
        widened += int(((fl & L.FLAG_WIDENED) != 0).sum().item())
        total += fl.numel()
        bands.append(float(st["band"].double().mean().item()))
    return {"hits": hits, "total": total, "rate": hits / total, "widened": widened, "seeds": trials,
            "mean_band": sum(bands) / len(bands)}


def miss_cost(L, torch, gen):
    """Forward times (ms, CUDA events, median) on the workload's rows: a
    bracket that holds, with and without the spread fallback (what the
    option costs when nothing misses), and a bracket forced to miss (below
    every score's b), solved by one workgroup's whole-row fallback or by the
    spread whole-row bucket solve."""
    import numpy as np
    w = workload(gen)
    r = torch.from_numpy(w.r).cuda()
    lo = float(np.min(w.r)) - 2.0
    cases = {"hit": (dict(path="bracket"), 5), "hit_spread": (dict(path="bracket", spread_fallback=True), 5),
             "miss_spread": (dict(path="bracket", bracket_override=(lo - 1.0, lo), spread_fallback=True), 3),
             "miss_one_workgroup": (dict(path="bracket", bracket_override=(lo - 1.0, lo)), 1)}
    out = {}
    for name, (opts, reps) in cases.items():
        L.lapsum_forward(r, w.k, w.t, **opts)  # warm-up
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            L.lapsum_forward(r, w.k, w.t, **opts)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        out[name + "_ms"] = float(np.median(times))
    out["note"] = ("forward only, one call per timing (workspace from the caching allocator); the forced "
                   "miss uses a bracket below every score")
    return out


def midpoint_drift(L, torch, gen):
    """DFTopK's fixed midpoint threshold on the workload's rows: the mass the
    Laplace kernel assigns there against k (LapSum's own threshold gives k)."""
    w = workload(gen)
    k = int(round(w.k))
    _, mass = L.midpoint_mass(torch.from_numpy(w.r).cuda(), k, w.t)
    rel = (mass / k - 1.0).cpu()
    return {"k": k, "mass_mean": float(mass.mean().item()), "drift_mean": float(rel.mean().item()),
            "drift_max_abs": float(rel.abs().max().item())}


def cpu_baseline(gen):
    """The oracle as it stands, timed on the host cores: forward (bisection)
    and forward + backward, median over runs; rows split across all cores for
    batches, one core for single rows, and for the 1e8 row a prefix sample
    with k scaled to keep k/n."""
    import numpy as np

    import oracle
    w = workload(gen)
    plan = CPU_PLAN[gen]
    threads = oracle.default_threads() if plan["threads"] == "all" else plan["threads"]
    r, g, k = w.r, w.g, w.k
    sample = f"all {w.rows}x{w.n} scores"
    if "prefix" in plan and plan["prefix"] < w.n:
        m = plan["prefix"]
        r = np.ascontiguousarray(w.r[:, :m])
        g = np.ascontiguousarray(w.g[:, :m])
        k = w.k * m / w.n
        sample = f"first {m} scores of the {w.n}-score row, k scaled to {k:g} (same k/n)"
    fwd, both = [], []
    for _ in range(plan["runs"]):
        t0 = time.perf_counter()
        _, b = oracle.forward(r, k, w.t, threads=threads)
        t1 = time.perf_counter()
        oracle.backward(r, b, g, w.t, threads=threads)
        t2 = time.perf_counter()
        fwd.append(t1 - t0)
        both.append(t2 - t0)
    elems = r.size
    fwd_s, both_s = sorted(fwd)[len(fwd) // 2], sorted(both)[len(both) // 2]
    return {"value": elems / both_s, "unit": "elements/s", "fwd_elements_per_s": elems / fwd_s, "cores": threads,
            "runs": plan["runs"], "kind": "oracle",
            "sample": f"{sample}, t={w.t}; fp64 bisection forward + analytic VJP, median of {plan['runs']} "
                      f"({both_s:.2f} s fwd+bwd)"}


def load_traffic(kernel_stage: str, workload_name: str):
    """Calibrated HBM bytes per launch from the committed counter summary, or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_stage}_{workload_name}.json")
    if not os.path.exists(path) or kernel_stage not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_sha") != source_sha(KERNEL_SOURCES[kernel_stage]):
        return None
    return tr.get("bytes_per_launch")


def comparisons(results):
    """The pages' relative-speed claims, re-measured here (forward only)."""
    out = {}

    def ratio(slow, fast):
        if slow in results and fast in results:
            return results[slow]["ms_fwd"] / results[fast]["ms_fwd"]
        return None
    pairs = {"bracket_vs_sort_1e8": ("extreme_sort", "extreme"),
             "bracket_vs_bucket_1e8": ("extreme_bucket", "extreme"),
             "sort_vs_bisect_1e8": ("extreme_bisect", "extreme_sort"),
             "bracket_vs_sort_32x65536": ("coder_sort", "coder_bracket"),
             "sort_vs_bisect_32x65536": ("coder_bisect", "coder_sort"),
             "bucket_vs_sort_32x65536": ("coder_sort", "coder_bucket")}
    for key, (slow, fast) in pairs.items():
        v = ratio(slow, fast)
        if v is not None:
            out[key] = {"speedup_fwd": v, "slower": slow, "faster": fast}
    out["pages"] = {"bracket_vs_full_sort_1e8": "up to 19x", "full_sort_vs_bisection": "nearly two orders of magnitude",
                    "note": "hardware, precision and workload not stated"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs", default=DEFAULT_CONFIGS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hit-trials", type=float, default=1.0,
                    help="scale of the planned hit-rate trial counts (0 skips them)")
    ap.add_argument("--no-miss-cost", action="store_true", help="skip the forced-miss forward timings")
    ap.add_argument("--calib-copy", action="store_true", help="also run a plain 1 GiB copy kernel (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 (no multi-GPU path exists)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_selection_primitive_amd as L
    L.load_library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hip = Hip()
    names = [c for c in args.configs.split(",") if c]
    results = {}
    head_name = "extreme" if "extreme" in names else names[0]
    for name in names:
        steps = args.steps if name.startswith("extreme") else max(args.steps, 1000)
        res = bench_workload(L, hip, torch, name, WORKLOADS[name], steps, args.warmup,
                             live_dominant=(name == head_name))
        # calibrated HBM bytes of the dominant kernel from the committed
        # counter summary (null when none matches the current sources)
        res["dominant"]["traffic"] = load_traffic(res["dominant"]["stage"], name)
        results[name] = res
        q = res["step_ms_quantiles"]
        print(f"# {name}: {res['fwd_bwd_elements_per_s']:.3e} el/s fwd+bwd, {res['ms_per_step']:.4f} ms/step "
              f"(median {q['median']:.4f}, p10 {q['p10']:.4f}, p90 {q['p90']:.4f}), "
              f"{100 * res['hbm_fraction_step']:.1f}% HBM (graph replay {res['ms_per_step_graph']:.4f} ms, "
              f"{100 * res['hbm_fraction_step_graph']:.1f}%), fwd {res['ms_fwd']:.4f} ms, dominant "
              f"{res['dominant']['stage']} {res['dominant']['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=bb)  # one elementwise kernel: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del a, bb

    gens = []
    for name in names:
        gen = WORKLOADS[name]["gen"]
        if gen not in gens:
            gens.append(gen)
    # bracketing hit rates (every configuration that brackets this generator's rows)
    if args.hit_trials > 0:
        for gen, trials in HIT_TRIALS.items():
            users = [nm for nm in names if WORKLOADS[nm]["gen"] == gen and results[nm]["path"] == "bracket"]
            if users:
                hr = hit_rate(L, torch, gen, max(1, int(round(trials * args.hit_trials))))
                for nm in users:
                    results[nm]["hit_rate"] = hr
                print(f"# hit rate {gen}: {hr['hits']}/{hr['total']}", file=sys.stderr, flush=True)
    # cost of a missed bracket, and of the spread fallback when nothing misses
    if not args.no_miss_cost:
        for gen in ("extreme", "attack"):
            users = [nm for nm in names if WORKLOADS[nm]["gen"] == gen and results[nm]["path"] == "bracket"]
            if users:
                mc = miss_cost(L, torch, gen)
                for nm in users:
                    results[nm]["miss_cost"] = mc
                print(f"# miss cost {gen}: " + ", ".join(f"{k} {v:.3f}" for k, v in mc.items() if k != "note"),
                      file=sys.stderr, flush=True)
    # DFTopK fixed-midpoint budget drift, per workload
    for gen in gens:
        md = midpoint_drift(L, torch, gen)
        for nm in names:
            if WORKLOADS[nm]["gen"] == gen and not WORKLOADS[nm].get("per_row"):
                results[nm]["dftopk_midpoint"] = md
        print(f"# DFTopK midpoint {gen}: mass/k - 1 = {md['drift_mean']:.3e}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    # the oracle on the host cores, per workload
    cpu_by_gen = {}
    if not args.no_cpu_baseline:
        for gen in gens:
            cpu_by_gen[gen] = cpu_baseline(gen)
            for nm in names:
                if WORKLOADS[nm]["gen"] == gen:
                    results[nm]["cpu_baseline"] = cpu_by_gen[gen]
            print(f"# oracle {gen}: {cpu_by_gen[gen]['value']:.3e} el/s fwd+bwd on {cpu_by_gen[gen]['cores']} cores",
                  file=sys.stderr, flush=True)

    head = results[head_name]
    sha = source_sha()
    dom = head["dominant"]
    traffic = load_traffic(dom["stage"], head_name)
    roofline = {"bound": "hbm", "achieved": dom["GBps"], "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": dom["GBps"] * 1e9 / HBM_PEAK, "traffic": traffic,
                "kernel": dom["kernel"], "algorithmic_bytes_per_launch": dom["bytes"],
                "avg_launch_ms": dom["avg_ms"], "step_frac": head["hbm_fraction_step"]}
    line = {
        "metric": "soft top-k elements/s fwd+bwd and % HBM roofline, n=3.3M and n=1e8, 1 GPU",
        "value": head["fwd_bwd_elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "rows": head["rows"], "n": head["n"], "k": head["k"],
                   "t": head["t"], "path": head["path"], "parallelism": "single GPU"},
        "hbm_fraction_step": head["hbm_fraction_step"],
        "roofline": roofline,
        "cpu_baseline": cpu_by_gen.get(WORKLOADS[head_name]["gen"]),
        "source_sha": sha,
        "pages_context": {"n": 100_000_000, "ms": 5.23,
                          "note": "hardware, precision, k, t, distribution and fwd/bwd not stated"},
        "comparisons": comparisons(results),
        "configs": results,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
