"""Benchmark of the MI355X Fast LapSum soft top-k (forward + backward).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs extreme,attack,...]

One step = one forward (threshold b and probabilities p) plus one backward
(dr, dk) over one batch, inputs resident in HBM.  The headline workload is
the single row of 1e8 scores (mixture 0.9 N(0,1) + 0.1 N(3, 0.5), k = 1e5,
t = 0.01, bracketing path); the other workloads are reported beside it.
Prints ONE JSON line.

Byte model (algorithmic bytes per score, what the method itself must move):
  on-chip rows:   fwd 8 (r in, p out), bwd 12 (g, p in, dr out)
  bracketing:     fwd 12 (r read by the filter pass and the apply pass, p out),
                  bwd 20 (g, p read twice, dr out: dk needs the whole row)
  full-sort rows: fwd 8 compulsory (sort traffic measured, not credited), bwd 20
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
                "bwd_apply": "bwd_apply_kernel", "band": "band_solve_onchip / segment_kernel",
                "select": "select_kernel", "sample": "sample_kernel", "fullsort": "segment_kernel",
                "init": "init_rows_kernel"}


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
    # name: (generator kwargs, path, bytes fwd, bytes bwd, steps scale)
    "extreme": dict(gen="extreme", path="auto", fwd_b=12, bwd_b=20),
    "attack": dict(gen="attack", path="auto", fwd_b=12, bwd_b=20),
    "routing": dict(gen="routing", path="auto", fwd_b=8, bwd_b=12),
    # the routing batch with a budget and a temperature per row (k_i in [2, 14],
    # t_i log-uniform in [0.02, 0.1], seed 4700)
    "routing_per_row": dict(gen="routing", path="auto", fwd_b=8, bwd_b=12, per_row=True),
    "coder_bracket": dict(gen="coder", path="bracket", fwd_b=12, bwd_b=20),
    "coder_fullsort": dict(gen="coder", path="fullsort", fwd_b=8, bwd_b=20),
    # the 1e8 row through the full-sort path (the pages compare bracketing
    # with a full sort at this size)
    "extreme_fullsort": dict(gen="extreme", path="fullsort", fwd_b=8, bwd_b=20),
    "tiny": dict(gen="tiny", path="auto", fwd_b=8, bwd_b=12),
}


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
    fwd = {L.PATH_ONCHIP: [L.STAGE_ONCHIP_FWD],
           L.PATH_FULLSORT: [L.STAGE_INIT, L.STAGE_FULLSORT, L.STAGE_APPLY],
           L.PATH_BRACKET: [L.STAGE_SAMPLE, L.STAGE_SELECT, L.STAGE_FILTER, L.STAGE_BAND,
                            L.STAGE_APPLY]}[path]  # the fallback runs inside the band stage
    bwd = [L.STAGE_ONCHIP_BWD] if n <= 1024 else [L.STAGE_BWD_REDUCE, L.STAGE_BWD_APPLY]
    return fwd + bwd


def bench_workload(L, hip, torch, name, spec, steps, warmup, seed=0, live_dominant=True):
    """live_dominant: time the dominant kernel with an event pair inside the
    timed region (the headline workload, run first); otherwise its time comes
    from the instrumented pass and the timed region records no event (event
    records were measured to turn into GPU round trips late in a long run of
    workloads, inflating their timed loops several times over)."""
    from sparse_selection_primitive_amd import workloads
    w = workloads.by_name(spec["gen"])
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
        import numpy as np
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
        for s in ran:
            ms = hip.elapsed_ms(evs[2 * s], evs[2 * s + 1])
            stage_ms.setdefault(L.STAGE_NAMES[s], []).append(ms)
        hip.destroy(evs)
    stage_avg = {k: sum(v) / len(v) for k, v in stage_ms.items()}
    dominant = max((k for k in stage_avg if k in STAGE_BYTES), key=lambda k: stage_avg[k])
    dom_id = L.STAGE_NAMES.index(dominant)

    # timed region: K steps, events only around the dominant kernel
    dom_events = [(hip.event(), hip.event()) for _ in range(steps)] if live_dominant else []
    ev_lists = []
    for a, b_ in dom_events:
        evs = [None] * (2 * L.STAGE_COUNT)
        evs[2 * dom_id], evs[2 * dom_id + 1] = a, b_
        ev_lists.append(evs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, ev_lists[i] if live_dominant else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if live_dominant:
        dom_ms = [hip.elapsed_ms(a, b_) for a, b_ in dom_events]
        hip.destroy([e for pair in dom_events for e in pair])
        dom_avg = sum(dom_ms) / len(dom_ms)
    else:
        dom_avg = stage_avg[dominant]

    # the same steps replayed from HIP graphs (one captured forward+backward
    # per buffer set): the launch cost of each kernel leaves the step
    graphs = []
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        for i in range(nsets):
            r, g, p, b, dr, dk = sets[i]
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap):
                cs = cap.cuda_stream
                op.forward(r, p, b, stream=cs)
                op.backward(g, p, b, dr, dk, stream=cs)
            graphs.append(gr)
    torch.cuda.current_stream(dev).wait_stream(cap)
    for i in range(max(warmup, nsets)):
        graphs[i % nsets].replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        graphs[i % nsets].replay()
    torch.cuda.synchronize()
    wall_graph = time.perf_counter() - t2
    del graphs

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
    ms_graph = 1e3 * wall_graph / steps
    step_bytes = (spec["fwd_b"] + spec["bwd_b"]) * elems
    dom_bytes = STAGE_BYTES[dominant] * elems
    out = {
        "workload": w.name, "rows": rows, "n": n, "k": w.k, "t": w.t, "path": ["auto", "onchip", "fullsort",
                                                                              "bracket"][plan["path"]],
        "fwd_bwd_elements_per_s": elems / (ms_step * 1e-3),
        "fwd_elements_per_s": elems / (ms_fwd * 1e-3),
        "ms_per_step": ms_step, "ms_fwd": ms_fwd,
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
    return out, w


def hit_rate(L, torch, name, path, trials):
    from sparse_selection_primitive_amd import workloads
    w = workloads.by_name(name)
    r = torch.from_numpy(w.r).cuda()
    hits = total = 0
    bands = []
    for seed in range(trials):
        _, _, st = L.lapsum_forward(r, w.k, w.t, path=path, seed=1000 + seed, stats=True)
        fl = st["flags"]
        hits += int(((fl & L.FLAG_HIT) != 0).sum().item())
        total += fl.numel()
        bands.append(float(st["band"].double().mean().item()))
    return {"hits": hits, "total": total, "rate": hits / total, "mean_band": sum(bands) / len(bands)}


def cpu_baseline(w_extreme_r, k, t, n_sample):
    """The oracle as it stands, on the first n_sample scores of the row with
    the budget scaled to keep k/n, forward (bisection) + backward."""
    import numpy as np

    import oracle
    r = np.ascontiguousarray(w_extreme_r[0, :n_sample])
    ks = k * n_sample / w_extreme_r.shape[1]
    g = np.random.Generator(np.random.PCG64(502)).standard_normal(n_sample).astype(np.float32)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    _, b = oracle.forward(r, ks, t, threads=threads)
    oracle.backward(r, b, g, t, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": n_sample / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_sample} scores of the 1e8 row, k scaled to {ks:g} (same k/n), t={t}; "
                      f"fp64 bisection forward + analytic VJP, {dt:.2f} s wall"}


def load_traffic(kernel_stage: str, workload: str):
    """Calibrated HBM bytes per launch from the committed counter summary, or
    None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_stage}_{workload}.json")
    if not os.path.exists(path) or kernel_stage not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_sha") != source_sha(KERNEL_SOURCES[kernel_stage]):
        return None
    return tr.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--configs",
                    default="extreme,attack,routing,routing_per_row,coder_bracket,coder_fullsort,extreme_fullsort,tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hit-trials", type=int, default=20)
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
    extreme_w = None
    head_name = "extreme" if "extreme" in names else names[0]
    for name in names:
        steps = args.steps if name.startswith("extreme") else max(args.steps, 100)
        res, w = bench_workload(L, hip, torch, name, WORKLOADS[name], steps, args.warmup,
                                live_dominant=(name == head_name))
        results[name] = res
        if name == "extreme":
            extreme_w = w
        print(f"# {name}: {res['fwd_bwd_elements_per_s']:.3e} el/s fwd+bwd, {res['ms_per_step']:.4f} ms/step, "
              f"{100 * res['hbm_fraction_step']:.1f}% HBM (graph replay {res['ms_per_step_graph']:.4f} ms, "
              f"{100 * res['hbm_fraction_step_graph']:.1f}%), dominant {res['dominant']['stage']} "
              f"{res['dominant']['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=bb)  # one elementwise kernel: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del a, bb

    hits = {}
    if args.hit_trials > 0:
        if "extreme" in names:
            hits["extreme"] = hit_rate(L, torch, "extreme", "auto", args.hit_trials)
        if "attack" in names:
            hits["attack"] = hit_rate(L, torch, "attack", "auto", 5 * args.hit_trials)
        if "coder_bracket" in names:
            hits["coder"] = hit_rate(L, torch, "coder", "bracket", args.hit_trials)
    for k_, v in hits.items():
        key = {"coder": "coder_bracket"}.get(k_, k_)
        if key in results:
            results[key]["hit_rate"] = v

    head = results[head_name]
    sha = source_sha()
    dom = head["dominant"]
    traffic = load_traffic(dom["stage"], head_name)
    roofline = {"bound": "hbm", "achieved": dom["GBps"], "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": dom["GBps"] * 1e9 / HBM_PEAK, "traffic": traffic,
                "kernel": dom["kernel"], "algorithmic_bytes_per_launch": dom["bytes"],
                "avg_launch_ms": dom["avg_ms"]}
    cpu = None
    if not args.no_cpu_baseline and extreme_w is not None:
        cpu = cpu_baseline(extreme_w.r, extreme_w.k, extreme_w.t, 20_000_000)
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
        "cpu_baseline": cpu,
        "source_sha": sha,
        "pages_context": {"n": 100_000_000, "ms": 5.23,
                          "note": "hardware, precision, k, t, distribution and fwd/bwd not stated"},
        "configs": results,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
