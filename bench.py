"""Benchmark: fused GEMM+AllReduce (one GPU's share) on MI355X.

A step is one call of the fused persistent kernel (mk_gemm_ar_local, adaptive
reducer count, default in-place policy) over one batch of synthetic inputs
already resident in HBM: C = A*B + the sum of the P-1 peer partials. The headline
workload is the largest shard (--workload large: M=N=K_local=8192, P=8; bf16
A/B/peers/C, fp32 accumulation), whose arithmetic intensity (819 flops per
compulsory byte) puts it on the matrix-core side of MI355X's ridge (about 312).
The two-kernel baseline (GEMM kernel, then reduce kernel) is timed in the same
process for the speedup.

Prints ONE JSON line. `value` is effective TFLOP/s = 2*M*N*K / time of the
headline call. `roofline` prices that kernel against its bound: matrix cores
(2.5 PFLOP/s bf16) at or above the ridge, HBM (8 TB/s, compulsory bytes A + B +
peers + C per launch) below it; achieved = algorithmic work per launch / average
launch time from HIP events on the launch stream. `workloads` times every other
workload the same way (fused and baseline, each with its own roofline), the mlp
shape also under the comparison schedules (two streams, CU-masked streams, every
tile handed over), and the GEMM+ReduceScatter and AllGather+GEMM shares.
cpu_baseline times the CPU oracle on a bounded sample of rows of the headline
workload.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload large]
                       [--headline-only] [--no-cpu-baseline]
       python bench.py --allgather       (the AllGather+GEMM share alone)
       python bench.py --all-configs     (one JSON line: every workload, fused /
                                          baseline / two-stream, median p10 p90)
       python bench.py --sweep large     (one JSON line: static reducer counts
                                          0..64 against the adaptive controller)
       python bench.py --cpu-oracle      (one JSON line: the CPU oracle's GFLOP/s on
                                          every workload and the host's threads)
       python bench.py --litmus 10000000 (one JSON line: flag hand-off latency and
                                          stale reads per protocol)
       python bench.py --peaks           (one JSON line: measured bf16 matrix-core
                                          and copy ceilings against published peaks)
       python bench.py --trace attn --trace-inplace 0
                                         (one JSON line: the controller's trace
                                          and the device-timer role breakdown)
       python bench.py --flag-overhead decode
                                         (one JSON line per flag scope: device
                                          timers of the tile-flag hand-over)

--all-configs times batches of calls between two HIP events (10 batches of 20
calls after warmup, the fused, baseline and two-stream batches alternating;
median, p10 and p90 of the per-call averages). Workloads
whose inputs are under 600 MB rotate through enough input sets to exceed 600 MB,
so that repeated calls do not find their peers in the 256 MB Infinity Cache.
"""
import argparse
import hashlib
import json
import re
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_{}.txt")
KERNEL_SOURCES = ["tile_gemm_all_amd/csrc/mk_kernels.hip", "tile_gemm_all_amd/csrc/mk_device.h",
                  "tile_gemm_all_amd/csrc/mk_controller.h"]


def code_only(text):
    """C/C++/HIP source without its comments and with runs of whitespace folded:
    what the compiler reads (string literals in these sources hold no comment
    markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sha():
    """Hash of the device sources' code (comments and layout left out), which the
    committed traffic counters are tied to."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken
    on the kernel source as it is now; else None."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha() or t.get("workload") != workload:
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(w, A, B, peers, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of rows of the workload."""
    import numpy as np
    import torch

    import mk_inputs
    import oracle

    Bb = mk_inputs.bits(B)
    threads = oracle.max_threads()

    def run_rows(rows):
        idx = torch.as_tensor(rows, device=A.device)
        Ab = mk_inputs.bits(A[idx])
        Pb = mk_inputs.bits(peers[:, idx, :])
        t0 = time.perf_counter()
        oracle.gemm_ar(Ab, Bb, Pb, w.c_dtype)
        return time.perf_counter() - t0

    probe = list(range(threads))
    t = run_rows(probe)
    n = int(max(threads, min(w.M, len(probe) * budget_s / max(t, 1e-3))))
    n = max(threads, (n // threads) * threads)
    rows = list(np.linspace(0, w.M - 1, n).astype(int))
    t = run_rows(rows)
    flops = 2.0 * len(rows) * w.N * w.K
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{len(rows)} of {w.M} rows of the {w.name} workload (all N={w.N}, "
                      f"K={w.K}, {w.n_peers} peers), fp64, {t:.1f} s"}


def _batched(legs, n_sets, stream, batches=10, per_batch=20, warmup=10):
    """Per-call averages of `batches` batches of `per_batch` calls for each leg
    (a name -> fn(input set) dict; call i of a leg uses input set i % n_sets),
    each batch between two events on `stream`. The legs' batches alternate, in
    an order rotated every batch, so that clock drift over the run falls on all
    legs alike."""
    import torch

    names = list(legs)
    for name in names:
        for i in range(warmup):
            legs[name](i % n_sets)
    torch.cuda.synchronize()
    times = {name: [] for name in names}
    i = 0
    for bi in range(batches):
        for j in range(len(names)):
            name = names[(bi + j) % len(names)]
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for k in range(per_batch):
                legs[name]((i + k) % n_sets)
            b.record(stream)
            torch.cuda.synchronize()
            times[name].append(a.elapsed_time(b) / per_batch * 1e3)  # us per call
        i += per_batch
    out = {}
    for name in names:
        v = sorted(times[name])
        pick = lambda q: v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
        out[name] = {"median_us": round(pick(0.5), 1), "p10_us": round(pick(0.1), 1),
                     "p90_us": round(pick(0.9), 1)}
    return out


def allgather(steps, warmup):
    """The AllGather+GEMM share on ag_up (rank 5) alone: baseline (gather kernel,
    then the GEMM kernel) and fused kernel in alternating batches; one JSON line.
    Short runs of it serve the kernels' counter passes."""
    import torch

    import mk_inputs
    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    aw = mk_inputs.AG_BY_NAME["ag_up"]
    shards, B = mk_inputs.make_ag_inputs(aw.Ms, aw.P, aw.N, aw.K, "gaussian", 1000 * aw.index,
                                         device="cuda")
    loc, peers = mk_inputs.shard_split(shards, 5)
    full = torch.empty((aw.M, aw.K), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((aw.M, aw.N), dtype=torch.bfloat16, device="cuda")
    r = _batched({"baseline": lambda i: mk.gemm_ag_baseline(loc, peers, full, B, C, 5),
                  "fused": lambda i: mk.gemm_ag_local(loc, peers, full, B, C, 5)},
                 1, stream, batches=4, per_batch=max(1, steps), warmup=warmup)
    mk.stream_status()
    print(json.dumps({"mode": "allgather", "workload": aw.name, "Ms": aw.Ms, "P": aw.P,
                      "N": aw.N, "K": aw.K, "rank": 5, **r,
                      "speedup": round(r["baseline"]["median_us"] / r["fused"]["median_us"], 4)}),
          flush=True)


def all_configs():
    import torch

    import mk_inputs
    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    res = {}
    for w in mk_inputs.WORKLOADS:
        n_sets = max(1, -(-600_000_000 // w.compulsory_bytes()))
        base = mk_inputs.workload_inputs(w, "gaussian", device="cuda")
        sets = [base] + [tuple(t.clone() for t in base) for _ in range(n_sets - 1)]
        cdt = torch.bfloat16 if w.c_dtype == "bf16" else torch.float32
        C = torch.empty((w.M, w.N), dtype=cdt, device="cuda")
        r = {"n_input_sets": n_sets}
        r.update(_batched({"fused": lambda i: mk.gemm_ar_local(*sets[i], C),
                           "baseline": lambda i: mk.gemm_then_reduce_baseline(*sets[i], C),
                           "two_stream": lambda i: mk.gemm_ar_two_stream(*sets[i], C)},
                          n_sets, stream))
        mk.stream_status()
        r["speedup_vs_baseline"] = round(r["baseline"]["median_us"] / r["fused"]["median_us"], 3)
        r["fused_TFLOPs"] = round(w.flops / (r["fused"]["median_us"] * 1e-6) / 1e12, 1)
        r["fused_GBps"] = round(w.compulsory_bytes() / (r["fused"]["median_us"] * 1e-6) / 1e9, 1)
        res[w.name] = r
        del sets, base, C
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "all-configs", "unit": "us per call", "results": res}), flush=True)


def sweep(name):
    """Static settings of the reducer target against the adaptive controller (the
    pages' Figure 3 style: each setting's time over the best static one), under
    dynamic hand-over (MK_OPT_INPLACE = -2): the target is the number of workgroups
    streaming a reduce at once, a tile is reduced in place by its workgroup while a
    slot is free and handed over otherwise. The default policy (every tile in place,
    or early reduce for few-tile shapes) and every tile handed over are timed beside
    it."""
    import torch

    import mk_inputs
    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    w = mk_inputs.BY_NAME[name]
    n_sets = max(1, -(-600_000_000 // w.compulsory_bytes()))
    base_in = mk_inputs.workload_inputs(w, "gaussian", device="cuda")
    sets = [base_in] + [tuple(t.clone() for t in base_in) for _ in range(n_sets - 1)]
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16 if w.c_dtype == "bf16" else torch.float32,
                    device="cuda")
    G = mk.fused_grid(*sets[0], C)
    per = 10 if w.flops > 1e10 else 100

    def t(nr):
        return _batched({"fused": lambda i: mk.gemm_ar_local(*sets[i], C, n_reduce_wg=nr)},
                        n_sets, stream, batches=5, per_batch=per,
                        warmup=3 * per)["fused"]["median_us"]

    # the knob: the reducer target under dynamic hand-over (MK_OPT_INPLACE = -2;
    # shapes with early reduce keep their schedule and sweep their reducer target)
    old = mk.get_option(mk.OPT_INPLACE)
    mk.set_option(mk.OPT_INPLACE, -2)
    static = {}
    try:
        for nr in sorted({0, 8, 16, 32, 64, 96, 128, 160, 192, 224, G - 1}):
            if nr < G:
                static[str(nr)] = t(nr)
        adaptive = t(None)
    finally:
        mk.set_option(mk.OPT_INPLACE, old)
    best = min(static.values())
    res = {"workload": name, "G": G, "unit": "us per call (median of 5 batches)",
           "static": static, "adaptive": adaptive, "best_static": best,
           "adaptive_over_best_static": round(adaptive / best, 4),
           "normalised": {k: round(v / best, 3) for k, v in static.items()}}
    res["default_policy_us"] = t(None)  # every tile in place (or early reduce)
    res["handover_all_us"] = None
    try:
        mk.set_option(mk.OPT_INPLACE, 0)
        res["handover_all_us"] = t(None)
    finally:
        mk.set_option(mk.OPT_INPLACE, old)
    mk.stream_status()
    print(json.dumps({"mode": "sweep", "results": res}), flush=True)


def trace(name, inplace):
    """One call with telemetry: the controller's trace (Figure 7 style: reducer
    target against compute and reduce progress) and the device-timer role
    breakdown."""
    import torch

    import mk_inputs
    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    w = mk_inputs.BY_NAME[name]
    A, B, peers = mk_inputs.workload_inputs(w, "gaussian", device="cuda")
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16 if w.c_dtype == "bf16" else torch.float32,
                    device="cuda")
    tel = torch.zeros(mk.TELEMETRY_BYTES, dtype=torch.uint8, device="cuda")
    old = mk.get_option(mk.OPT_INPLACE)
    mk.set_option(mk.OPT_INPLACE, inplace)
    try:
        for _ in range(3):
            mk.gemm_ar_local(A, B, peers, C, telemetry=tel)
        mk.stream_status()
    finally:
        mk.set_option(mk.OPT_INPLACE, old)
    t = mk.Telemetry.from_buffer_copy(bytes(tel.cpu().numpy()))
    span = (t.t_end - t.t_start) / 100.0  # us (100 MHz ticks)
    slots = t.grid * span
    pts = [{"t_us": round((t.trace[i].t - t.t_start) / 100.0, 1), "computed": t.trace[i].computed,
            "reduced": t.trace[i].reduced, "target": t.trace[i].target,
            "streaming": t.trace[i].spare} for i in range(t.n_trace)]
    print(json.dumps({"mode": "trace", "workload": name, "inplace_option": inplace,
                      "span_us": round(span, 1), "grid": t.grid, "tiles": t.tiles,
                      "busy_compute_frac": round(t.busy_compute / 100.0 / slots, 3),
                      "busy_reduce_frac": round(t.busy_reduce / 100.0 / slots, 3),
                      "wait_reduce_frac": round(t.wait_reduce / 100.0 / slots, 3),
                      "initial_target": t.initial_target, "final_target": t.final_target,
                      "updates": t.n_updates, "trace": pts}), flush=True)


def flag_overhead(name):
    """Tile-flag overhead inside the fused kernel, from its device timers: every tile
    handed to reducers through its flag (MK_OPT_INPLACE=0; 128x128 tiles on shapes
    that would otherwise take 64x64 ones, which never publish), under XCD-local
    flags (scope 0) and agent-scope release/acquire (scope 1). Per published tile:
    ticks from its partial's store-complete wait to its flag store; per reduce
    unit: ticks from the poll that sees the flag to the end of the acquire. One
    JSON line per scope, with the call's time without telemetry next to it."""
    import torch

    import mk_inputs
    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    w = mk_inputs.BY_NAME[name]
    A, B, peers = mk_inputs.workload_inputs(w, "gaussian", device="cuda")
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16 if w.c_dtype == "bf16" else torch.float32,
                    device="cuda")
    tel = torch.zeros(mk.TELEMETRY_BYTES, dtype=torch.uint8, device="cuda")
    opts = (mk.OPT_INPLACE, mk.OPT_FLAG_SCOPE, mk.OPT_TILE_SHAPE)
    old = [mk.get_option(o) for o in opts]
    tiles128 = -(-w.M // 128) * -(-w.N // 128)
    shape = 2 if tiles128 < torch.cuda.get_device_properties(0).multi_processor_count else 0
    try:
        for scope in (0, 1):
            mk.set_option(mk.OPT_INPLACE, 0)
            mk.set_option(mk.OPT_FLAG_SCOPE, scope)
            mk.set_option(mk.OPT_TILE_SHAPE, shape)
            for _ in range(3):
                mk.gemm_ar_local(A, B, peers, C, telemetry=tel)
            mk.stream_status()
            t = mk.Telemetry.from_buffer_copy(bytes(tel.cpu().numpy()))
            reps = 50 if w.flops < 1e10 else 10
            for _ in range(3):
                mk.gemm_ar_local(A, B, peers, C)
            torch.cuda.synchronize()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                mk.gemm_ar_local(A, B, peers, C)
            ev1.record(stream)
            torch.cuda.synchronize()
            mk.stream_status()
            span = (t.t_end - t.t_start) / 100.0  # us (100 MHz ticks)
            slots = t.grid * span
            print(json.dumps({
                "mode": "flag_overhead", "workload": name, "flag_scope": scope,
                "tile": "128x128" if shape == 2 else "auto", "tiles": t.tiles, "grid": t.grid,
                "call_us": round(ev0.elapsed_time(ev1) / reps * 1e3, 2),
                "span_us_with_telemetry": round(span, 2),
                "published": t.published,
                "publish_us_per_tile": round(t.publish_ticks / 100.0 / max(t.published, 1), 3),
                "acquired": t.acquired,
                "acquire_us_per_unit": round(t.acquire_ticks / 100.0 / max(t.acquired, 1), 3),
                "publish_frac_of_workgroup_time": round(t.publish_ticks / 100.0 / slots, 4),
                "acquire_frac_of_workgroup_time": round(t.acquire_ticks / 100.0 / slots, 4),
                "wait_reduce_frac": round(t.wait_reduce / 100.0 / slots, 4)}), flush=True)
    finally:
        for o, v in zip(opts, old):
            mk.set_option(o, v)


def peaks():
    """Measured ceilings of the chip next to the published ones the rooflines use:
    bf16 matrix-core throughput of register-only MFMA chains on every compute unit
    (mk_mfma_peak) and the bandwidth of a plain elementwise copy (read + write)."""
    import torch

    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    stream = torch.cuda.current_stream()

    def timed_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
    iters = 20000
    ms = timed_ms(lambda: mk.mfma_peak(iters, cus, out))
    mk.stream_status()
    flops = cus * 4 * 8 * iters * 32768
    tf = flops / (ms * 1e-3) / 1e12
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda").uniform_()
    y = torch.empty_like(x)
    cms = timed_ms(lambda: torch.neg(x, out=y), reps=10)
    gbps = 2 * x.numel() * 4 / (cms * 1e-3) / 1e9
    print(json.dumps({
        "mode": "peaks", "device": props.name, "compute_units": cus,
        "mfma_bf16": {"TFLOPs": round(tf, 1), "published_dense_TFLOPs": BF16_PEAK_TFLOPS,
                      "frac_of_published": round(tf / BF16_PEAK_TFLOPS, 3),
                      "workgroups": cus, "iters": iters, "ms": round(ms, 3)},
        "copy": {"GBps": round(gbps, 1), "published_GBps": HBM_PEAK_GBPS,
                 "frac_of_published": round(gbps / HBM_PEAK_GBPS, 3),
                 "bytes_each_way": x.numel() * 4, "ms": round(cms, 3)},
    }), flush=True)


def litmus(n):
    """The tile-flag message-passing litmus (mk_flag_handoff) n times for each
    protocol, on one XCD and across two: ns per hand-off and stale data reads."""
    import torch

    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    res = []
    for scope, name in ((2, "fused protocol (stores complete, relaxed flag, agent acquire)"),
                        (1, "agent-scope release/acquire"),
                        (0, "workgroup-scope invalidate only")):
        for cross in (False, True):
            left, ns_sum, stale, xcds = n, 0.0, 0, None
            while left > 0:  # calls of at most 2^24 hand-offs
                k = min(left, 1 << 24)
                ns, st, xcds = mk.flag_handoff(k, scope, cross)
                ns_sum += ns * k
                stale += st
                left -= k
            res.append({"protocol": name, "flag_scope": scope, "xcds": list(xcds),
                        "trials": n, "ns_per_handoff": round(ns_sum / n, 1), "stale": stale})
    print(json.dumps({"mode": "litmus", "results": res}), flush=True)


def cpu_oracle(budget_s=8.0):
    """The cpu_baseline leg for every workload: the CPU oracle's throughput with
    all host threads (rows
    sampled evenly to about budget_s seconds where the whole shard would take
    longer), and one thread for the tiny and decode shards (whole shard)."""
    import numpy as np

    import mk_inputs
    import oracle

    threads = oracle.max_threads()
    res = {}
    for w in mk_inputs.WORKLOADS:
        A, B, peers = mk_inputs.workload_inputs(w, "gaussian", device="cpu")
        Bb = mk_inputs.bits(B)

        def run_rows(rows, nthreads):
            Ab = mk_inputs.bits(A[rows])
            Pb = mk_inputs.bits(peers[:, rows, :])
            t0 = time.perf_counter()
            oracle.gemm_ar(Ab, Bb, Pb, w.c_dtype, threads=nthreads)
            return time.perf_counter() - t0

        r = {}
        for nthreads in ([threads, 1] if w.name in ("tiny", "decode") else [threads]):
            probe = list(range(min(w.M, max(nthreads, 8))))
            t = run_rows(probe, nthreads)
            n = int(min(w.M, len(probe) * budget_s / max(t, 1e-4)))
            n = max(len(probe), n)
            rows = sorted(set(np.linspace(0, w.M - 1, n).astype(int).tolist()))
            t = run_rows(rows, nthreads)
            r[f"threads_{nthreads}"] = {
                "GFLOPs": round(2.0 * len(rows) * w.N * w.K / t / 1e9, 2),
                "rows": len(rows), "of_rows": w.M, "seconds": round(t, 2)}
        res[w.name] = r
        del A, B, peers
    print(json.dumps({"mode": "cpu-oracle", "host_threads": threads, "results": res}),
          flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)  # flops per byte, about 312


def roofline_of(w, us):
    """The bound of a workload's fused call (matrix cores at or above the ridge,
    HBM below it) and the fraction of that peak the call reaches: algorithmic
    flops or compulsory bytes per launch over the launch time."""
    if w.flops / w.compulsory_bytes() >= RIDGE:
        tf = w.flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    gbps = w.compulsory_bytes() / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large",
                    help="the workload of the headline line (default: the largest, 8192^3)")
    ap.add_argument("--n-reduce-wg", type=int, default=None,
                    help="static reducer count (default: adaptive controller)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload's fused call and its baseline")
    ap.add_argument("--all-configs", action="store_true")
    ap.add_argument("--allgather", action="store_true",
                    help="the AllGather+GEMM share alone (baseline and fused, alternating)")
    ap.add_argument("--sweep", metavar="WORKLOAD")
    ap.add_argument("--trace", metavar="WORKLOAD",
                    help="one call with telemetry; --trace-inplace 0 hands every tile over")
    ap.add_argument("--trace-inplace", type=int, default=-1)
    ap.add_argument("--flag-overhead", metavar="WORKLOAD",
                    help="device timers of the tile-flag hand-over (publish and acquire) "
                         "with every tile handed over, under both flag scopes")
    ap.add_argument("--cpu-oracle", action="store_true",
                    help="the CPU oracle's GFLOP/s on every workload (all threads; one "
                         "thread for tiny and decode)")
    ap.add_argument("--litmus", type=int, metavar="N",
                    help="flag message-passing litmus, N hand-offs per protocol and placement")
    ap.add_argument("--peaks", action="store_true",
                    help="measured ceilings: bf16 matrix-core TFLOP/s and copy GB/s")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the fused kernel and has no multi-GPU "
              "mode (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.all_configs:
        all_configs()
        return
    if args.allgather:
        allgather(args.steps, args.warmup)
        return
    if args.sweep:
        sweep(args.sweep)
        return
    if args.trace:
        trace(args.trace, args.trace_inplace)
        return
    if args.flag_overhead:
        flag_overhead(args.flag_overhead)
        return
    if args.litmus:
        litmus(args.litmus)
        return
    if args.cpu_oracle:
        cpu_oracle()
        return
    if args.peaks:
        peaks()
        return

    import torch

    import mk_inputs
    import tile_gemm_all_amd as mk

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    w = mk_inputs.BY_NAME[args.workload]

    def new_c(wl):
        return torch.empty((wl.M, wl.N), dtype=torch.bfloat16 if wl.c_dtype == "bf16" else
                           torch.float32, device="cuda")

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        mk.stream_status()
        return start.elapsed_time(stop) / steps  # ms per launch

    def timed_pair(fb, ff, steps, warmup, rounds=4):
        """Baseline and fused legs of one comparison, timed in alternating blocks
        (b f f b b f f b): the clock of a power-limited chip drifts over a run, and
        two legs timed one after the other would carry that drift into their ratio.
        Returns the median block time of each leg, ms per launch."""
        for _ in range(warmup):
            fb()
            ff()
        per = max(1, -(-steps // rounds))
        tb, tf = [], []
        for r in range(rounds):
            for leg in ((0, 1) if r % 2 == 0 else (1, 0)):
                (tb if leg == 0 else tf).append(timed(fb if leg == 0 else ff, per, 0))
        return statistics.median(tb), statistics.median(tf)

    # Comparison legs get at least 50 warmup calls: the first leg timed in a fresh
    # process ran several percent slow after 10 (two-kernel baseline on mlp:
    # 0.336 ms after 10, 0.322 ms after 100, on one box), which would flatter the
    # fused kernel. The headline's fused leg, timed last, keeps --warmup.
    cw = max(args.warmup, 50)
    out_workloads = {}
    extras = {}
    if not args.headline_only:
        # every other workload: fused (adaptive) and two-kernel baseline, inputs
        # rotated over enough sets that the peers are not cache-resident
        for o in mk_inputs.WORKLOADS:
            if o.name == w.name:
                continue
            n_sets = max(1, -(-600_000_000 // o.compulsory_bytes()))
            base_in = mk_inputs.workload_inputs(o, "gaussian", device="cuda")
            sets = [base_in] + [tuple(t.clone() for t in base_in) for _ in range(n_sets - 1)]
            C = new_c(o)
            it = [0]

            def rot(fn):
                def call():
                    fn(*sets[it[0] % n_sets], C)
                    it[0] += 1
                return call

            steps = max(args.steps, 20 if o.flops > 1e10 else 200)
            b_ms, f_ms = timed_pair(rot(mk.gemm_then_reduce_baseline), rot(mk.gemm_ar_local),
                                    steps, cw)
            r = {"M": o.M, "N": o.N, "K_local": o.K, "P": o.P, "input_sets": n_sets,
                 "fused_us": round(f_ms * 1e3, 2), "baseline_us": round(b_ms * 1e3, 2),
                 "speedup_vs_two_kernel": round(b_ms / f_ms, 4),
                 "TFLOPs": round(o.flops / (f_ms * 1e-3) / 1e12, 2),
                 "GBps": round(o.compulsory_bytes() / (f_ms * 1e-3) / 1e9, 1),
                 "roofline": roofline_of(o, f_ms * 1e3),
                 "schedule": mk.SCHEDULES[mk.fused_schedule(*sets[0], C)]}
            if o.name == "mlp":
                A, B, peers = base_in
                # the comparison schedules of the pages' Figure 1 on the mlp shape
                r["two_stream_us"] = round(timed(lambda: mk.gemm_ar_two_stream(A, B, peers, C),
                                                 args.steps, cw) * 1e3, 2)
                masked = {}
                n_cus = mk.num_workgroups()
                old_split = mk.get_option(mk.OPT_STREAM_CU_SPLIT)
                try:
                    for split in range(n_cus // 4, n_cus, n_cus // 4):
                        mk.set_option(mk.OPT_STREAM_CU_SPLIT, split)
                        masked[str(split)] = round(timed(
                            lambda: mk.gemm_ar_two_stream(A, B, peers, C), args.steps, cw) * 1e3, 1)
                finally:
                    mk.set_option(mk.OPT_STREAM_CU_SPLIT, old_split)
                r["two_stream_cu_masked_us"] = {"by_reduce_cus": masked,
                                               "best": min(masked.values()) if masked else None}
                # the role-split path alone: every tile handed to reducers by its flag
                old_inplace = mk.get_option(mk.OPT_INPLACE)
                mk.set_option(mk.OPT_INPLACE, 0)
                try:
                    r["handover_all_us"] = round(timed(lambda: mk.gemm_ar_local(A, B, peers, C),
                                                       args.steps, cw) * 1e3, 2)
                finally:
                    mk.set_option(mk.OPT_INPLACE, old_inplace)
                # GEMM+ReduceScatter share of the same GEMM: this GPU owns one P-th of
                # the rows (slice 3), reduces them with the peers' partials of those
                # rows and publishes the rest
                o0, o1 = 3 * o.M // o.P, 4 * o.M // o.P
                rs_peers = peers[:, o0:o1].contiguous()
                rs_C = torch.empty((o1 - o0, o.N), dtype=C.dtype, device="cuda")
                rs_send = torch.empty((o.M, o.N), dtype=peers.dtype, device="cuda")
                rs_b, rs_f = timed_pair(
                    lambda: mk.gemm_rs_baseline(A, B, rs_peers, rs_C, rs_send, o0, o1),
                    lambda: mk.gemm_rs_local(A, B, rs_peers, rs_C, rs_send, o0, o1),
                    args.steps, cw)
                extras["reduce_scatter"] = {"workload": "mlp GEMM", "owned_rows": [o0, o1],
                                            "fused_us": round(rs_f * 1e3, 2),
                                            "baseline_us": round(rs_b * 1e3, 2),
                                            "speedup": round(rs_b / rs_f, 4)}
                del rs_peers, rs_C, rs_send
            out_workloads[o.name] = r
            del sets, base_in, C
            torch.cuda.empty_cache()
        # AllGather+GEMM share (gate+up projection, column-parallel): this GPU (rank
        # 5) holds 256 of the 4096 gathered rows; the other 15 shards land while the
        # GEMM runs
        aw = mk_inputs.AG_BY_NAME["ag_up"]
        ag_shards, ag_B = mk_inputs.make_ag_inputs(aw.Ms, aw.P, aw.N, aw.K, "gaussian",
                                                   1000 * aw.index, device="cuda")
        ag_local, ag_peers = mk_inputs.shard_split(ag_shards, 5)
        del ag_shards
        ag_full = torch.empty((aw.M, aw.K), dtype=torch.bfloat16, device="cuda")
        ag_C = torch.empty((aw.M, aw.N), dtype=torch.bfloat16, device="cuda")
        ag_b, ag_f = timed_pair(
            lambda: mk.gemm_ag_baseline(ag_local, ag_peers, ag_full, ag_B, ag_C, 5),
            lambda: mk.gemm_ag_local(ag_local, ag_peers, ag_full, ag_B, ag_C, 5),
            args.steps, cw)
        extras["allgather"] = {"workload": f"{aw.name}: {aw.description}", "Ms": aw.Ms,
                               "P": aw.P, "N": aw.N, "K": aw.K, "rank": 5,
                               "fused_us": round(ag_f * 1e3, 2),
                               "baseline_us": round(ag_b * 1e3, 2),
                               "speedup": round(ag_b / ag_f, 4),
                               "fused_TFLOPs": round(aw.flops / (ag_f * 1e-3) / 1e12, 2)}
        del ag_local, ag_peers, ag_full, ag_B, ag_C
        torch.cuda.empty_cache()

    # the headline workload, timed last: its fused calls are the last dispatches of
    # the run
    A, B, peers = mk_inputs.workload_inputs(w, "gaussian", device="cuda")
    C = new_c(w)
    base_ms = timed(lambda: mk.gemm_then_reduce_baseline(A, B, peers, C), args.steps, cw)
    t0 = time.perf_counter()
    fused_ms = timed(lambda: mk.gemm_ar_local(A, B, peers, C, n_reduce_wg=args.n_reduce_wg),
                     args.steps, args.warmup)
    wall = time.perf_counter() - t0

    tflops = w.flops / (fused_ms * 1e-3) / 1e12
    roofline = roofline_of(w, fused_ms * 1e3)
    roofline["traffic"] = measured_traffic(w.name)
    out = {
        "metric": "fused GEMM+reduce TFLOP/s, % MFMA/HBM roofline, speedup vs 2-kernel baseline",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fused_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "M": w.M, "N": w.N, "K_local": w.K,
                   "P": w.P, "peer_dtype": w.peer_dtype, "c_dtype": w.c_dtype,
                   "reducers": "adaptive" if args.n_reduce_wg is None else args.n_reduce_wg,
                   # the adaptive call's schedule: with every tile reduced in place the
                   # controller keeps no dedicated reducers (a static count takes the
                   # role split instead)
                   "schedule": (mk.SCHEDULES[mk.fused_schedule(A, B, peers, C)]
                                if args.n_reduce_wg is None
                                else f"persistent kernel, {args.n_reduce_wg} workgroups prefer "
                                     "reducing")},
        "roofline": roofline,
        "effective_GBps": round(w.compulsory_bytes() / (fused_ms * 1e-3) / 1e9, 1),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "two_kernel_ms": round(base_ms, 5),
        "speedup_vs_two_kernel": round(base_ms / fused_ms, 4),
        "workloads": out_workloads,
        "timed_wall_s": round(wall, 3),
    }
    out.update(extras)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A, B, peers)
    print(json.dumps(out), flush=True)
    # free the library's workspaces (and the streams they own) before the process
    # exits; the library also does this itself at exit
    mk.workspace_reset()


if __name__ == "__main__":
    main()
