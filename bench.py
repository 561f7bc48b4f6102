"""Throughput of the Adasum combine on one MI355X.

One step is one full combine (every tree level of every segment) of the
K gradient buffers of a synthetic workload that is already resident in HBM.
Default workload: the BERT-Large-shaped set, K = 16 fp32 gradients of
335,141,888 parameters in 391 segments.

Prints one JSON line: gradient GB/s (K * N * bytes per element / step time),
the HBM-roofline figures of the dominant kernel (from HIP events around every
launch inside the timed region) and of the whole path (minimum traffic of
reading K gradients once and writing one), and the fp64 CPU oracle timed on a
bounded sample of the same workload, against which the GPU result of that
sample is checked ("parity").
"""

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gradient GB/s combined (K·bytes/time) and % of HBM roofline, 1 MI355X"
PEAK_HBM_GBS = 8000.0
WORKLOAD_NAMES = {1: "small_k2_f32", 2: "resnet50_k8_f32", 3: "bert_large_k16_f32",
                  4: "bert_base_k64_f16", 5: "stress_20k_k32_bf16"}
BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "distributed_sgd_gradient_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def host_threads():
    """Host cores the oracle may use: this process's CPU affinity, at most 16
    (a one-GPU share of a shared host, whatever the machine's core count)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


TOL_REL_L2 = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
TOL_COEFF = 1e-6


def cpu_baseline(wl, budget_s, schedule="tree", threads=1, batch_bytes=8 << 30, gpu_out=None, gpu_coeffs=None):
    """Time the fp64 oracle (the same schedule as the GPU run, the oracle's
    own code unchanged) on whole segments copied from the GPU workload.

    Pass 1, one thread: segments are added (largest-first order of the layer
    list) until the budget is spent.  Pass 2, the same segments on a pool of
    `threads` threads, one segment per task, largest first, fetched in
    batches of at most `batch_bytes` of fp64 data (fetches are not timed).
    NumPy releases the GIL in the oracle's dot products and array
    arithmetic; every BLAS call runs on one thread.

    Outside the timed calls, pass 1 also compares the GPU result `gpu_out`
    and coefficients `gpu_coeffs` ([K-1][nseg][2]) with the oracle's on every
    sampled segment.  Returns (baseline record, parity record or None)."""
    import concurrent.futures

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    fn = oracle.adasum_chain if schedule == "chain" else oracle.adasum_tree
    first = min(5, wl.nseg)  # encoder layers first, the (large) embedding segments last
    order = list(range(first, wl.nseg)) + list(range(0, first))
    used, elems, spent = [], 0, 0.0
    err2 = ref2 = 0.0
    cerr = 0.0
    exempt = unsettled_segments = 0
    coeffs_host = gpu_coeffs.cpu().numpy() if gpu_coeffs is not None else None
    with threadpool_limits(limits=1):
        for s in order:
            rows = wl.segment_host(s)
            t0 = time.perf_counter()
            res, coeffs, stats = fn(rows)
            spent += time.perf_counter() - t0
            used.append(s)
            elems += rows[0].size
            if gpu_out is not None or coeffs_host is not None:
                # outside the timed call: which coefficients, and whether this
                # segment's output, the oracle itself determines (one-ulp noise
                # on the inputs moves them by less than a tenth of their
                # tolerance); the rest is reported, not gated
                stab = oracle.stability(rows, [0, rows[0].size], schedule)
                seg_ok = stab["output_motion"][0] <= TOL_REL_L2[wl.dtype] / 10
                unsettled_segments += 0 if seg_ok else 1
            if gpu_out is not None and seg_ok:
                lo, hi = int(wl.seg_offsets[s]), int(wl.seg_offsets[s + 1])
                ref = oracle.round_to_format(res, wl.dtype)
                got = gpu_out[lo:hi].double().cpu().numpy()
                err2 += float(np.sum((got - ref) ** 2))
                ref2 += float(np.sum(ref ** 2))
            if coeffs_host is not None and len(coeffs):
                c = np.asarray(coeffs, dtype=np.float64)
                zero = stab["coeff_motion"][:, 0, :] > TOL_COEFF / 10
                exempt += int(np.count_nonzero(zero))
                err = np.where(zero, 0.0, np.abs(coeffs_host[:, s, :] - c) / np.maximum(1.0, np.abs(c)))
                cerr = max(cerr, float(np.max(err)))
            del rows, res
            if spent >= budget_s:
                break
        pooled = spent
        if threads > 1:
            pooled = 0.0
            seg_len = lambda s: int(wl.seg_offsets[s + 1] - wl.seg_offsets[s])  # noqa: E731
            todo = sorted(used, key=seg_len, reverse=True)
            with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
                while todo:
                    batch, size = [], 0
                    while todo and (not batch or size + seg_len(todo[0]) * wl.K * 8 <= batch_bytes):
                        size += seg_len(todo[0]) * wl.K * 8
                        batch.append(wl.segment_host(todo.pop(0)))
                    t0 = time.perf_counter()
                    for _ in ex.map(fn, batch):
                        pass
                    pooled += time.perf_counter() - t0
                    del batch
    nbytes = wl.K * elems * BYTES[wl.dtype]
    base = {"value": nbytes / pooled / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(used)} of {wl.nseg} segments ({elems} of {wl.N} elements per worker); "
                      f"{threads} threads of fp64 NumPy, one segment per task, one BLAS thread each",
            "seconds": pooled, "cpu_model": cpu_model(),
            "one_core": {"value": nbytes / spent / 1e9, "unit": "GB/s", "seconds": spent}}
    parity = None
    if gpu_out is not None:
        rel = (err2 ** 0.5) / (ref2 ** 0.5) if ref2 > 0 else (0.0 if err2 == 0 else float("inf"))
        tol = TOL_REL_L2[wl.dtype]
        parity = {"against": "fp64 oracle, rounded to the output dtype", "segments": len(used),
                  "elements_per_worker": elems, "rel_l2": rel, "tol_rel_l2": tol,
                  "max_coeff_err": cerr if coeffs_host is not None else None, "tol_coeff": TOL_COEFF,
                  "coeffs_not_determined_by_the_oracle": exempt if coeffs_host is not None else None,
                  "segments_not_determined_by_the_oracle": unsettled_segments,
                  "pass": bool(rel <= tol and (coeffs_host is None or cerr <= TOL_COEFF))}
    return base, parity


def time_steps(step, steps, profile):
    """Run `steps` combines back to back on the current stream, bracketed by
    synchronisations.  Returns (mean ms per step from the host clock, the
    per-step GPU times from events recorded at every step boundary on the
    launch stream, per-kernel rows of HIP events around every launch or
    None)."""
    import torch

    from distributed_sgd_gradient_amd import _native

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if profile:
        _native.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernels = _native.profile_end() if profile else None
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return (t1 - t0) * 1e3 / steps, per_step, kernels


def time_bare(step, steps):
    """Mean ms per step of `steps` combines back to back with no event inside
    the loop (host clock, bracketed by synchronisations)."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_graph(step, steps, per_graph=10):
    """Mean ms per step when `per_graph` combines are captured into one HIP
    graph and the graph is replayed: the same kernels without the host's
    launch cost (the earlier calls have uploaded the shape's tables)."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            step()
    reps = max(1, steps // per_graph)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * per_graph)
    del g
    return ms


def step_stats(ms, per_step):
    srt = sorted(per_step)
    return {"mean": ms, "median": srt[len(srt) // 2], "min": srt[0], "max": srt[-1]}


def kernel_table(kernels, steps):
    return {k: {"launches": v["launches"], "ms_per_step": v["milliseconds"] / steps,
                "bytes_per_step": v["bytes"] / steps,
                "achieved_GBps": v["bytes"] / (v["milliseconds"] * 1e-3) / 1e9 if v["milliseconds"] > 0 else 0.0,
                "frac": (v["bytes"] / (v["milliseconds"] * 1e-3) / 1e9 / PEAK_HBM_GBS
                         if v["milliseconds"] > 0 else 0.0)} for k, v in kernels.items()}


def other_workload(config, steps, warmup, dev, budget_s):
    """A compact record of another workload in the same run: step time
    (mean, median, min), path roofline, per-kernel times and parity against
    the oracle on a bounded sample of its segments."""
    import torch

    import distributed_sgd_gradient_amd as A
    import workloads as W

    log(f"other workload {config} ({WORKLOAD_NAMES[config]})")
    wl = W.make_workload(config, device=dev)
    K, N, esz = wl.K, wl.N, BYTES[wl.dtype]
    if N < 1 << 22:
        steps = max(steps, 200)  # a launch-bound combine of a few microseconds: more steps for a stable figure
    out = torch.empty_like(wl.grads[0])
    step = A.Combiner(wl.grads, wl.seg_offsets, out=out, return_coeffs=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms, per_step, _ = time_steps(step, steps, profile=False)  # events at step boundaries only
    _, _, kernels = time_steps(step, steps, profile=True)     # per-kernel times, a pass of its own
    b_min = K * N * esz + N * esz
    st = step_stats(ms, per_step)
    log(f"  {steps} steps: {ms:.3f} ms/step (median {st['median']:.3f}, min {st['min']:.3f})")
    bare = time_bare(step, steps)
    graph = time_graph(step, steps)
    log(f"  without events: {bare * 1e3:.1f} us/step; graph replay: {graph * 1e3:.1f} us/step")
    _, parity = cpu_baseline(wl, budget_s, "tree", 1, gpu_out=out, gpu_coeffs=step.coeffs)
    log(f"  parity on {parity['segments']} segments: relative L2 {parity['rel_l2']:.3g}, "
        f"coefficient error {parity['max_coeff_err']}")
    rec = {"workload": WORKLOAD_NAMES[config], "K": K, "N": N, "nseg": wl.nseg, "io_dtype": wl.dtype,
           "ms_per_step": st, "ms_per_step_without_events": bare, "ms_per_step_graph_replay": graph,
           "gradient_GBps": K * N * esz / (ms * 1e-3) / 1e9,
           "path_frac": b_min / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "B_min_bytes": b_min,
           "kernels": kernel_table(kernels, steps), "parity": parity}
    del step, out, wl
    torch.cuda.empty_cache()
    return rec


def _median_ms(fn, reps=5):
    """Median of `reps` timed calls of fn (HIP events on the current stream)."""
    import torch

    fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return sorted(ms)[len(ms) // 2]


def probe(name, dev):
    """Measurements behind design decisions, run with the library's own
    kernels (one JSON line per case):

    cache  - the K = 16 fp32 plain sum of one group of buffers repeated 32
             times in a HIP graph (its inputs were just read: the memory-side
             cache can serve them) against 32 different groups in turn, for
             groups of 8 MiB to 512 MiB of inputs;
    groups - the combine of 2^26 elements per worker (K = 16 fp32) as one
             call, against the same segments cut into groups combined one
             after another (a HIP graph of all groups, on one stream and
             alternating over two), so that each group's second read could
             come from the memory-side cache;
    seggroups - the same interleaving on the BERT-Large workload itself:
             runs of consecutive segments whose K-operand footprint fits a
             cap (64, 136 or 256 MiB) are packed into groups of at most the
             cap, runs of larger segments are one call each, and the calls
             replay one after another in a HIP graph (one stream, and
             alternating over two), against the workload as one call;
             printed with the step times, the number of calls and the
             share of the input bytes that sits in groups;
    launch - back-to-back plain sums of 8 elements (K = 1) in a graph: the
             cost of a dependent launch;
    host   - the small K = 2 workload (two launches per combine): host time
             per eager `Combiner` call, per call of the C entry point with
             marshalled arguments, and per `torch.cuda.current_stream()`
             lookup, beside the GPU time per combine with no event in the
             loop and as graph replays: whether such combines are bound by
             the host or by the GPU."""
    import torch

    import distributed_sgd_gradient_amd as A

    K, T = 16, 1 << 26
    out_lines = []
    if name in ("cache", "groups"):
        gen = torch.Generator(device=dev).manual_seed(5)
        big = [torch.randn(T, device=dev, generator=gen) for _ in range(K)]
        out = torch.empty(T, device=dev)
    if name == "cache":
        R = 32
        for lg in range(17, 24):
            ng = 1 << lg
            ngroups = T // ng
            sl = [slice((g % ngroups) * ng, (g % ngroups + 1) * ng) for g in range(R)]
            A.plain_sum([b[sl[0]] for b in big], out=out[sl[0]])
            torch.cuda.synchronize()
            same, cyc = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(same):
                for _ in range(R):
                    A.plain_sum([b[sl[0]] for b in big], out=out[sl[0]])
            with torch.cuda.graph(cyc):
                for r in range(R):
                    A.plain_sum([b[sl[r]] for b in big], out=out[sl[r]])
            t_same, t_cyc = _median_ms(same.replay) / R, _median_ms(cyc.replay) / R
            nbytes = (K + 1) * ng * 4
            out_lines.append({"probe": "cache", "input_MiB": K * ng * 4 >> 20, "same_group_us": t_same * 1e3,
                              "same_group_GBps": nbytes / (t_same * 1e-3) / 1e9, "groups_in_turn": min(ngroups, R),
                              "in_turn_us": t_cyc * 1e3, "in_turn_GBps": nbytes / (t_cyc * 1e-3) / 1e9})
            del same, cyc
    elif name == "groups":
        bmin = (K + 1) * T * 4
        for lg in (19, 21, 23):
            ng, nper = 1 << lg, 4
            ngroups = T // ng
            off = [i * (ng // nper) for i in range(ngroups * nper + 1)]
            whole = A.Combiner(big, off, out=out)
            t_whole = _median_ms(whole)
            del whole
            groups = []
            for g in range(ngroups):
                sl = slice(g * ng, (g + 1) * ng)
                groups.append(A.Combiner([b[sl] for b in big], [i * (ng // nper) for i in range(nper + 1)],
                                         out=out[sl]))
            for c in groups:
                c()
            torch.cuda.synchronize()
            one, two = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(one):
                for c in groups:
                    c()
            side = torch.cuda.Stream()
            with torch.cuda.graph(two):
                cur = torch.cuda.current_stream()
                side.wait_stream(cur)
                for i, c in enumerate(groups):
                    if i % 2:
                        with torch.cuda.stream(side):
                            c()
                    else:
                        c()
                cur.wait_stream(side)
            t_one, t_two = _median_ms(one.replay), _median_ms(two.replay)
            out_lines.append({"probe": "groups", "group_input_MiB": K * ng * 4 >> 20, "groups": ngroups,
                              "one_call_ms": t_whole, "groups_one_stream_ms": t_one, "groups_two_streams_ms": t_two,
                              "one_call_path_frac": bmin / (t_whole * 1e-3) / 1e9 / PEAK_HBM_GBS})
            del one, two, groups
            torch.cuda.synchronize()
    elif name == "seggroups":
        import workloads as W

        wl = W.make_workload(3, device=dev)
        grads, off = wl.grads, [int(x) for x in wl.seg_offsets]
        K, nseg, N = len(grads), len(off) - 1, off[-1]
        esz = grads[0].element_size()
        bmin = (K + 1) * N * esz
        out = torch.empty_like(grads[0])
        ref = torch.empty_like(grads[0])
        whole = A.Combiner(grads, off, out=ref)
        whole()
        torch.cuda.synchronize()
        for cap_mib in (64, 136, 256):
            cap = cap_mib << 20
            fits = [K * esz * (off[s + 1] - off[s]) <= cap for s in range(nseg)]
            runs, s = [], 0
            while s < nseg:
                e = s + 1
                if fits[s]:
                    while e < nseg and fits[e] and K * esz * (off[e + 1] - off[s]) <= cap:
                        e += 1
                else:
                    while e < nseg and not fits[e]:
                        e += 1
                runs.append((s, e, fits[s]))
                s = e
            calls = []
            for s, e, _ in runs:
                lo, hi = off[s], off[e]
                if lo % 4:  # 16-byte aligned bases only (every BERT tensor holds a multiple of 4 elements)
                    raise SystemExit("segment group not 16-byte aligned")
                calls.append(A.Combiner([g[lo:hi] for g in grads], [x - lo for x in off[s:e + 1]], out=out[lo:hi]))
            for c in calls:
                c()
            torch.cuda.synchronize()
            diff = ((out.double() - ref.double()).norm() / ref.double().norm()).item()
            one, two = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(one):
                for c in calls:
                    c()
            side = torch.cuda.Stream()
            with torch.cuda.graph(two):
                cur = torch.cuda.current_stream()
                side.wait_stream(cur)
                for i, c in enumerate(calls):
                    if i % 2:
                        with torch.cuda.stream(side):
                            c()
                    else:
                        c()
                cur.wait_stream(side)
            wg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(wg):
                whole()
            t = {"whole": [], "one": [], "two": []}
            for _ in range(5):  # alternating, so that a drift of the box's rate hits all three alike
                t["whole"].append(_median_ms(wg.replay, 3))
                t["one"].append(_median_ms(one.replay, 3))
                t["two"].append(_median_ms(two.replay, 3))
            med = {k: sorted(v)[len(v) // 2] for k, v in t.items()}
            grouped = sum(off[e] - off[s] for s, e, f in runs if f)
            out_lines.append({"probe": "seggroups", "workload": WORKLOAD_NAMES[3], "cap_MiB": cap_mib,
                              "calls": len(calls), "grouped_calls": sum(1 for r in runs if r[2]),
                              "grouped_byte_share": grouped / N, "one_call_ms": med["whole"],
                              "groups_one_stream_ms": med["one"], "groups_two_streams_ms": med["two"],
                              "one_call_path_frac": bmin / (med["whole"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                              "rel_l2_vs_one_call": diff})
            print(json.dumps(out_lines[-1]), flush=True)
            del one, two, wg, calls
            torch.cuda.synchronize()
        out_lines = []
    elif name == "launch":
        x = torch.ones(8, device=dev)
        y = torch.empty_like(x)
        A.plain_sum([x], out=y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(100):
                A.plain_sum([x], out=y)
        out_lines.append({"probe": "launch", "us_per_dependent_launch": _median_ms(g.replay) * 10})
    elif name == "host":
        import ctypes

        import workloads as W

        wl = W.make_workload(1, device=dev)
        out = torch.empty_like(wl.grads[0])
        step = A.Combiner(wl.grads, wl.seg_offsets, out=out, return_coeffs=True)
        step()
        torch.cuda.synchronize()
        st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

        def host_us(fn, n):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            t1 = time.perf_counter()
            torch.cuda.synchronize()
            return (t1 - t0) / n * 1e6

        rec = {"probe": "host", "workload": WORKLOAD_NAMES[1]}
        for _ in range(2):  # the second pass is reported
            rec["combiner_call_us"] = host_us(step, 200)
            rec["c_entry_call_us"] = host_us(lambda: step._fn(*step._args, st), 200)
            rec["current_stream_lookup_us"] = host_us(lambda: torch.cuda.current_stream(dev), 2000)
            rec["gpu_us_without_events"] = time_bare(step, 200) * 1e3
            rec["gpu_us_graph_replay"] = time_graph(step, 200) * 1e3
        out_lines.append(rec)
    else:
        raise SystemExit(f"unknown probe {name!r} (cache, groups, seggroups, launch, host)")
    for ln in out_lines:
        print(json.dumps(ln), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--schedule", choices=["tree", "chain"], default="tree",
                    help="order of the pairwise combines: the tree (default) or the left-to-right chain")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of one-thread oracle time that bound the CPU baseline's sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--others", default="1,2,4",
                    help="comma-separated workloads also timed in the same run (compact records under "
                         "'other_workloads'); only with the default workload; '' for none")
    ap.add_argument("--cold", action="store_true",
                    help="also time each step alone after writing a 1 GiB scratch buffer (caches cold); "
                         "reported under 'cold', the headline value stays the back-to-back rate")
    ap.add_argument("--probe", choices=["cache", "groups", "seggroups", "launch", "host"], default=None,
                    help="instead of the benchmark, print the measurements behind a design decision (see probe())")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 3 plain fp32 copies of MIB MiB (read MIB, write MIB) "
                         "so that rocprofv3 counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the combine has no multi-GPU path", file=sys.stderr, flush=True)
        sys.exit(1)

    import torch

    import distributed_sgd_gradient_amd as A
    import workloads as W

    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", "0")))
    torch.cuda.set_device(dev)
    if args.probe:
        probe(args.probe, dev)
        return
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 3}))
        return
    log(f"generating workload {args.config} ({WORKLOAD_NAMES[args.config]}) on {dev}")
    wl = W.make_workload(args.config, seed=args.seed, device=dev)
    K, N, esz = wl.K, wl.N, BYTES[wl.dtype]
    out = torch.empty_like(wl.grads[0])
    # marshalled once; the coefficient table is written by every combine anyway
    step = A.Combiner(wl.grads, wl.seg_offsets, schedule=args.schedule, out=out, return_coeffs=True)
    torch.cuda.synchronize()

    log(f"K={K} N={N} nseg={wl.nseg}; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: the steps bracketed by synchronisations, a HIP event
    # at every step boundary (per-step times) and none inside a step
    ms, per_step, _ = time_steps(step, args.steps, profile=False)
    steps_ms = step_stats(ms, per_step)
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (median {steps_ms['median']:.3f}, min {steps_ms['min']:.3f})")
    # the same steps again with HIP events around every launch on the launch
    # stream: the per-kernel times behind the roofline
    ms_ev, per_step_ev, kernels = time_steps(step, args.steps, profile=True)
    ev_ms = step_stats(ms_ev, per_step_ev)
    log(f"again with per-launch events (per-kernel times): {ms_ev:.3f} ms/step (median {ev_ms['median']:.3f})")
    ms_noev = time_bare(step, args.steps)
    ms_graph = time_graph(step, args.steps)
    log(f"again without any event in the loop: {ms_noev * 1e3:.1f} us/step; "
        f"as HIP graph replays: {ms_graph * 1e3:.1f} us/step")

    grad_bytes = K * N * esz
    b_min = grad_bytes + N * esz
    value = grad_bytes / (ms * 1e-3) / 1e9
    dom_name = max(kernels, key=lambda k: kernels[k]["milliseconds"])
    dom = kernels[dom_name]
    per_launch_ms = dom["milliseconds"] / dom["launches"]
    per_launch_bytes = dom["bytes"] / dom["launches"]
    achieved = per_launch_bytes / (per_launch_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(WORKLOAD_NAMES[args.config], dom_name),
                "kernel": dom_name, "launch_ms": per_launch_ms, "algorithmic_bytes_per_launch": per_launch_bytes,
                "scope": f"the dominant kernel ({dom_name}) alone; the whole path's fraction of the HBM "
                         f"roofline, the metric's figure, is path_roofline.frac"}
    path = {"B_min_bytes": b_min, "achieved": b_min / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": b_min / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "frac_median_step": b_min / (steps_ms["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    for name, k in sorted(kernels.items()):
        log(f"  {name:12s} launches {k['launches']:5d}  {k['milliseconds'] / args.steps:8.3f} ms/step  "
            f"{k['bytes'] / (k['milliseconds'] * 1e-3) / 1e9 if k['milliseconds'] > 0 else 0:8.1f} GB/s")

    cold = None
    if args.cold:
        # each step alone, after a 1 GiB write has pushed the inputs out of
        # the L2 and Infinity caches; events on the stream the combine uses
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        times = []
        for _ in range(args.steps):
            scratch.fill_(1.0)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            step()
            ev1.record()
            ev1.synchronize()
            times.append(ev0.elapsed_time(ev1))
        del scratch
        cold_ms = float(sorted(times)[len(times) // 2])
        cold = {"ms_per_step_median": cold_ms, "ms_per_step_min": float(min(times)),
                "gradient_GBps": grad_bytes / (cold_ms * 1e-3) / 1e9,
                "path_frac": b_min / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "note": "one step at a time after a 1 GiB scratch write"}
        log(f"cold (caches flushed before every step): median {cold_ms:.3f} ms/step")

    # the synchronous-SGD plain sum on the same buffers: one pass, reads K
    # gradients once and writes one result (B_min of traffic)
    out_sum = torch.empty_like(out)
    for _ in range(args.warmup):
        A.plain_sum(wl.grads, out=out_sum)
    torch.cuda.synchronize()
    sum_ms, sum_steps, _ = time_steps(lambda: A.plain_sum(wl.grads, out=out_sum), args.steps, profile=False)
    plain_sum = {"ms_per_step": sum_ms, "ms_per_step_median": sorted(sum_steps)[len(sum_steps) // 2],
                 "gradient_GBps": grad_bytes / (sum_ms * 1e-3) / 1e9,
                 "path_frac": b_min / (sum_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "adasum_over_sum_time": ms / sum_ms}
    log(f"plain sum on the same buffers: {sum_ms:.3f} ms/step; Adasum takes {ms / sum_ms:.2f}x as long")
    del out_sum

    cpu = parity = None
    if not args.no_cpu_baseline:
        threads = host_threads()
        log(f"timing the CPU oracle on a sample (~{args.cpu_budget:.0f} s on one thread, then on {threads}); "
            f"the last timed step's result is checked against it")
        cpu, parity = cpu_baseline(wl, args.cpu_budget, args.schedule, threads, gpu_out=out,
                                   gpu_coeffs=step.coeffs)
        log(f"parity on {parity['segments']} segments: relative L2 {parity['rel_l2']:.3g}, "
            f"coefficient error {parity['max_coeff_err']}")

    config = {"workload": WORKLOAD_NAMES[args.config], "K": K, "N": N, "nseg": wl.nseg, "io_dtype": wl.dtype,
              "seed": wl.seed, "schedule": args.schedule, "parallelism": "none (one GPU)"}
    others = {}
    if args.others and args.config == 3 and args.seed is None and args.schedule == "tree":
        del step, wl
        torch.cuda.empty_cache()
        for c in [int(x) for x in args.others.split(",") if x]:
            others[WORKLOAD_NAMES[c]] = other_workload(c, args.steps, args.warmup, dev,
                                                       0.0 if args.no_cpu_baseline else 5.0)

    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": config,
        "roofline": roofline, "path_roofline": path, "cpu_baseline": cpu, "parity": parity,
        "step_ms": steps_ms, "step_ms_with_launch_events": ev_ms,
        "step_ms_without_events": ms_noev, "step_ms_graph_replay": ms_graph, "plain_sum": plain_sum,
        **({"cold": cold} if cold is not None else {}),
        "kernels": kernel_table(kernels, args.steps),
        **({"other_workloads": others} if others else {}),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
